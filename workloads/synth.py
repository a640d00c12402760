"""Seeded synthetic inputs for the verification step.

Every workload here is synthetic: the pages measure on WMT En-De and CNN/DM
with T5 checkpoints, which are not available, so Gaussian logit rows with the
shapes and overlap levels of the benchmark configurations stand in for them.

This module produces inputs only (logits, drafted tokens, uniforms).  It holds
none of the verification arithmetic: drafted tokens are drawn by the Gumbel-max
trick (argmax of logits/T plus Gumbel noise), which never forms a softmax or a
cumulative sum.

bf16 tensors are carried as uint16 arrays of raw bits (round-to-nearest-even
from float32).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .philox import uniforms as philox_uniforms

# Philox tags: separate counter streams for separate purposes.
TAG_UNIFORMS = 0x5EC0


@dataclasses.dataclass
class VerifyCase:
    """One verification problem: everything spec_verify consumes."""

    name: str
    target: np.ndarray      # [B, gamma+1, V] float32, or uint16 bf16 bits
    draft: np.ndarray       # [B, gamma, V]   same dtype as target
    dtype: str              # "f32" or "bf16"
    tokens: np.ndarray      # int32 [B, gamma]
    uniforms: np.ndarray    # float32 [B, gamma+1]
    temperature: float

    @property
    def B(self) -> int:
        return self.target.shape[0]

    @property
    def gamma(self) -> int:
        return self.target.shape[1] - 1

    @property
    def V(self) -> int:
        return self.target.shape[2]

    def subset(self, seqs) -> "VerifyCase":
        seqs = np.asarray(seqs)
        return VerifyCase(self.name, self.target[seqs], self.draft[seqs], self.dtype,
                          self.tokens[seqs], self.uniforms[seqs], self.temperature)


# ---------------------------------------------------------------- helpers

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.

    Works in chunks of 4M values with in-place operations, so gigabyte-sized
    weight matrices convert without gigabyte-sized temporaries.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(b.shape, dtype=np.uint16)
    chunk = 1 << 22
    t = np.empty(min(chunk, b.size), dtype=np.uint32)
    for lo in range(0, b.size, chunk):
        src = b[lo:lo + chunk]
        tt = t[:src.size]
        np.right_shift(src, np.uint32(16), out=tt)
        np.bitwise_and(tt, np.uint32(1), out=tt)
        np.add(tt, np.uint32(0x7FFF), out=tt)
        np.add(tt, src, out=tt)
        np.right_shift(tt, np.uint32(16), out=tt)
        out[lo:lo + src.size] = tt
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(logits: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(logits) if dtype == "bf16" else np.asarray(logits, np.float32)


def gumbel_max_tokens(draft_f32: np.ndarray, temperature: float, rng: np.random.Generator) -> np.ndarray:
    """Draft tokens x ~ softmax(draft/T) via Gumbel-max; x = argmax(draft) at T = 0.

    draft_f32: [B, gamma, V].  Processed one sequence at a time to bound memory.
    """
    B, G, V = draft_f32.shape
    out = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        rows = draft_f32[b].astype(np.float64)
        if temperature == 0.0:
            out[b] = np.argmax(rows, axis=-1)
        else:
            u = rng.random((G, V))
            u = np.clip(u, 1e-300, None)
            g = -np.log(-np.log(u))
            out[b] = np.argmax(rows / temperature + g, axis=-1)
    return out


def make_uniforms(seed: int, B: int, gamma: int, offsets=None) -> np.ndarray:
    return philox_uniforms(seed, B, gamma + 1, offsets=offsets, tag=TAG_UNIFORMS)


def _finish(name, target32, draft32, dtype, temperature, seed, offsets=None) -> VerifyCase:
    if dtype == "bf16":
        target = f32_to_bf16_bits(target32)
        draft = f32_to_bf16_bits(draft32)
    else:
        target = np.ascontiguousarray(target32, dtype=np.float32)
        draft = np.ascontiguousarray(draft32, dtype=np.float32)
    rng = np.random.default_rng([seed, 0x70CE])
    tokens = gumbel_max_tokens(as_f32(draft, dtype), temperature, rng)
    B, G1, _ = target.shape
    u = make_uniforms(seed, B, G1 - 1, offsets)
    return VerifyCase(name, target, draft, dtype, tokens, u, float(temperature))


# ------------------------------------------------------- generic workload

def gaussian_case(B: int, gamma: int, V: int, dtype: str = "f32", temperature: float = 1.0,
                  seed: int = 0, target_std: float = 2.0, draft_scale: float = 1.0,
                  draft_noise: float = 1.0, name: str = "gauss") -> VerifyCase:
    """Target ~ N(0, target_std^2) i.i.d.; draft = draft_scale * target + N(0, draft_noise^2).

    Draft row i uses target row i (i < gamma), the position the draft proposed for.
    """
    rng = np.random.default_rng([seed, 0x10])
    target = (rng.standard_normal((B, gamma + 1, V), dtype=np.float32) * np.float32(target_std))
    noise = rng.standard_normal((B, gamma, V), dtype=np.float32) * np.float32(draft_noise)
    draft = np.float32(draft_scale) * target[:, :gamma] + noise
    return _finish(name, target, draft, dtype, temperature, seed)


# ------------------------------------------------ the benchmark configurations

def config1(seed: int = 0, temperature: float = 1.0) -> VerifyCase:
    """B=1, gamma=3, V=32128, fp32: target ~ N(0, 2^2); draft = target + N(0, 1)."""
    return gaussian_case(1, 3, 32128, "f32", temperature, seed, 2.0, 1.0, 1.0, name="cfg1")


def config2(seed: int = 0, temperature: float = 1.0, rounds: int = 1) -> VerifyCase:
    """B=rounds, gamma=7, V=32128, fp32: target ~ N(0, 3^2); draft = 0.8 target + N(0, 0.5^2).

    Each batch row is one independent round with fresh logits.
    """
    return gaussian_case(rounds, 7, 32128, "f32", temperature, seed, 3.0, 0.8, 0.5, name="cfg2")


def _per_sequence(name: str, B: int, gamma: int, V: int, dtype: str, temperature: float, seed: int, tag: int,
                  make_rows, offsets=None, workers: int = 8) -> VerifyCase:
    """A batch built one sequence at a time on worker threads (numpy's
    generators release the interpreter lock).  make_rows(rng, b) returns the
    float32 target [gamma+1, V] and draft [gamma, V] rows of sequence b from
    rng, a stream of its own spawned from (seed, tag); its drafted tokens come
    from another stream of its own spawned from (seed, 0x70CE).  The result
    depends only on the seed and the shape, never on `workers`."""
    rows_ss = np.random.SeedSequence([seed, tag]).spawn(B)
    tok_ss = np.random.SeedSequence([seed, 0x70CE]).spawn(B)
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, gamma + 1, V), dtype=store)
    draft = np.empty((B, gamma, V), dtype=store)
    tokens = np.zeros((B, gamma), dtype=np.int32)

    def work(b):
        t32, d32 = make_rows(np.random.default_rng(rows_ss[b]), b)
        if dtype == "bf16":
            target[b] = f32_to_bf16_bits(t32)
            draft[b] = f32_to_bf16_bits(d32)
        else:
            target[b], draft[b] = t32, d32
        tokens[b] = gumbel_max_tokens(as_f32(draft[b:b + 1], dtype), temperature,
                                      np.random.default_rng(tok_ss[b]))[0]

    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(work, range(B)))
    u = make_uniforms(seed, B, gamma, offsets)
    return VerifyCase(name, target, draft, dtype, tokens, u, float(temperature))


def config3(seed: int = 0, temperature: float = 1.0, B: int = 64, V: int = 128256) -> VerifyCase:
    """B=64, gamma=4, V=128256, bf16.

    Target ~ N(0, 3^2) with 8 distinct random tokens per target row raised by +8;
    draft = target + N(0, sigma_b^2) with sigma_b ~ U(0.2, 2.0) per sequence; each
    sequence draws its uniforms from its own Philox counter offset.
    """
    gamma = 4
    rng = np.random.default_rng([seed, 0x30])
    sigma = rng.uniform(0.2, 2.0, size=B).astype(np.float32)
    offsets = rng.integers(0, 2 ** 32, size=B, dtype=np.uint64)

    def rows(r, b):
        t = r.standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(3.0)
        for i in range(gamma + 1):
            t[i, r.choice(V, size=min(8, V), replace=False)] += np.float32(8.0)
        d = t[:gamma] + r.standard_normal((gamma, V), dtype=np.float32) * sigma[b]
        return t, d

    return _per_sequence("cfg3", B, gamma, V, "bf16", temperature, seed, 0x31, rows, offsets)


def config5(seed: int = 0, temperature: float = 1.0, B: int = 256, V: int = 256000,
            wrong_fraction: float = 0.05) -> VerifyCase:
    """B=256, gamma=8, V=256000, bf16.

    Target ~ N(0, 4^2) plus a Zipf(1.1)-ranked bias -1.1 ln(rank), with one random
    rank-to-token permutation per seed shared by every row.  Draft = target + N(0, 1.5^2).
    In a seeded 5% of draft rows the draft is confidently wrong: the token the
    target rates lowest gets the draft row's maximum + 20.
    """
    gamma = 8
    rng = np.random.default_rng([seed, 0x50])
    perm = rng.permutation(V)
    bias = np.empty(V, dtype=np.float32)
    bias[perm] = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    wrong = rng.random((B, gamma)) < wrong_fraction
    offsets = rng.integers(0, 2 ** 32, size=B, dtype=np.uint64)

    def rows(r, b):
        t = r.standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(4.0)
        t += bias
        d = t[:gamma] + r.standard_normal((gamma, V), dtype=np.float32) * np.float32(1.5)
        for i in np.nonzero(wrong[b])[0]:
            d[i, int(np.argmin(t[i]))] = d[i].max() + np.float32(20.0)
        return t, d

    return _per_sequence("cfg5", B, gamma, V, "bf16", temperature, seed, 0x51, rows, offsets)


@dataclasses.dataclass
class LMHeadCase:
    """Inputs of the fused LM-head + verify workload (bf16 bits as uint16)."""

    hidden: np.ndarray      # [B*(gamma+1), d]
    w_target: np.ndarray    # [d, V]
    w_draft: np.ndarray     # [d, V]
    B: int
    gamma: int
    tokens: np.ndarray      # int32 [B, gamma]
    uniforms: np.ndarray    # float32 [B, gamma+1]
    temperature: float

    @property
    def d(self) -> int:
        return self.hidden.shape[1]

    @property
    def V(self) -> int:
        return self.w_target.shape[1]

    def draft_hidden_rows(self) -> np.ndarray:
        """Row indices of `hidden` the draft head reads: positions 0..gamma-1 of each sequence."""
        g1 = self.gamma + 1
        return np.array([b * g1 + i for b in range(self.B) for i in range(self.gamma)], dtype=np.int64)


def _normal_bf16_weights(seed: int, d: int, V: int, std: float, noise_std: float,
                         blocks: int = 32, workers: int = 8):
    """W_p ~ N(0, std^2) and W_q = W_p + N(0, noise_std^2), both [d, V] bf16 bits.

    The rows are cut into `blocks` blocks; block j draws from its own stream
    spawned from (seed, 0x40) and is converted on a worker thread (numpy's
    generators release the GIL), so a gigabyte matrix takes seconds.  The
    result depends only on the seed and the shape, never on `workers`.
    """
    children = np.random.SeedSequence([seed, 0x40]).spawn(blocks)
    wp = np.empty((d, V), dtype=np.uint16)
    wq = np.empty((d, V), dtype=np.uint16)
    bounds = [(j * d // blocks, (j + 1) * d // blocks) for j in range(blocks)]

    def work(j):
        lo, hi = bounds[j]
        if hi <= lo:
            return
        rng = np.random.default_rng(children[j])
        p32 = rng.standard_normal((hi - lo, V), dtype=np.float32)
        p32 *= np.float32(std)
        n32 = rng.standard_normal((hi - lo, V), dtype=np.float32)
        n32 *= np.float32(noise_std)
        n32 += p32
        wp[lo:hi] = f32_to_bf16_bits(p32)
        wq[lo:hi] = f32_to_bf16_bits(n32)

    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(work, range(blocks)))
    return wp, wq


def config4(seed: int = 0, temperature: float = 1.0, B: int = 8, gamma: int = 4,
            d: int = 4096, V: int = 128256) -> LMHeadCase:
    """Fused LM head + verify: hidden [B(gamma+1), d] ~ N(0,1); W_p ~ N(0, 0.02^2);
    W_q = W_p + N(0, 0.005^2); all bf16.

    Drafted tokens are Gumbel-max samples from the draft head's own fp32 logits,
    as the draft model would have produced them.
    """
    rng = np.random.default_rng([seed, 0x41])
    M = B * (gamma + 1)
    hidden = f32_to_bf16_bits(rng.standard_normal((M, d), dtype=np.float32))
    wp, wq = _normal_bf16_weights(seed, d, V, 0.02, 0.005)
    case = LMHeadCase(hidden, wp, wq, B, gamma, np.zeros((B, gamma), np.int32),
                      make_uniforms(seed, B, gamma), float(temperature))
    hq = bf16_bits_to_f32(hidden[case.draft_hidden_rows()])
    draft_logits = np.zeros((B * gamma, V), dtype=np.float32)
    for lo in range(0, d, 512):
        draft_logits += hq[:, lo:lo + 512] @ bf16_bits_to_f32(wq[lo:lo + 512])
    case.tokens = gumbel_max_tokens(draft_logits.reshape(B, gamma, V), temperature,
                                    np.random.default_rng([seed, 0x70CE]))
    return case


CONFIGS = {1: config1, 2: config2, 3: config3, 5: config5}
