"""Plain fp64 NumPy oracle of the verification step.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the bench's
CPU-baseline leg.  Page abbreviations are listed in oracle/__init__.py.

The step, per sequence, with positions indexed from 0 (target rows p_0..p_gamma,
draft rows q_0..q_{gamma-1}, drafted tokens x_0..x_{gamma-1}):

  1. p_i = softmax(target_i / T), q_i = softmax(draft_i / T); temperature is applied
     to both models ([FI] "The loop: draft, verify in one pass, keep a prefix";
     [NZ] "5. Sampling and evaluation").  T = 0 means argmax, a one-hot
     distribution ([FI] "Speculative sampling: the accept/reject rule", last
     paragraphs on temperature).
  2. Overlap alpha_i = sum_x min(p_i, q_i) = 1 - TV(p_i, q_i) for every draft
     position ([SD] "How often do we accept?"; [FI] "The acceptance rate is the
     overlap of p and q", Lemma 3.3).
  3. Walk the drafts left to right: keep x_i when u_i <= min(1, p_i(x_i)/q_i(x_i)),
     stop at the first failure; n = number kept ([FI] Algorithm 1, steps 3-4;
     [SD] "The algorithm").
  4. If n < gamma, sample from the residual max(0, p_n - q_n) normalised by its
     sum; otherwise sample the bonus token from p_gamma ([FI] Algorithm 1 step 4
     and eq. (2); [SD] "Exactness").
  5. The sample uses its own uniform u_gamma and the inverse CDF in token-index
     order: the first token whose cumulative weight exceeds u_gamma.

Readings taken where the pages are silent (each is listed in the design notes):
  * u_gamma is a fresh uniform for the final sample; the rejecting u_n is not reused.
  * `sample()` is the inverse CDF with a strict ">" in token-index order.
  * A residual with no mass falls back to p_n ([LH] "Three candidates explain
    the acceptance rule": a zero-mass residual is never normalised).  In exact
    arithmetic that needs p_n = q_n, where only a draft outside the support
    (0/0) is rejected.  Any positive mass, however small, is sampled.
  * Argmax ties go to the lowest token index; alpha in argmax mode is the
    indicator that the two argmaxes agree.
  * alpha is reported for every draft position, whatever n is.
  * p/q uses IEEE semantics: q(x) = 0 < p(x) gives +inf (accept); 0/0 gives NaN,
    and any comparison with NaN is false (reject).

Two extensions, both off by default:
  * Lenience l in (0, 1] ([FI] "The acceptance rate is the overlap of p and q",
    the paragraph on the lenience factor of Appendix A.5): q(x) is multiplied by
    l before the comparison, so x is kept when u <= min(1, p(x) / (l q(x))).  The
    page does not give the residual under l; the reading taken here builds it
    from the same scaled comparison, max(0, p - l q).  With that residual no
    token is emitted more than 1/l times as often as under p (the bound the page
    states), and l = 1 is the exact method.
  * Per-sequence draft counts gamma_b <= gamma (a dynamic lookahead, [LH] "A
    longer draft is not always faster"): sequence b's data sit in positions 0..gamma_b of the
    padded arrays (drafts 0..gamma_b-1, target rows 0..gamma_b, accept uniforms
    0..gamma_b-1, final-sample uniform u[b][gamma_b]); positions past gamma_b are
    padding, never read, and report alpha = p(x) = q(x) = NaN.  gamma_b = 0 is a
    plain decoding step: the token is sampled from p_0.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses

import numpy as np

from oracle import adjust

# |u_i - min(1, p_i(x_i)/q_i(x_i))| below this marks an accept decision that
# other arithmetic may take differently; such sequences are flagged (u_band).
U_BAND = 1e-6


# ------------------------------------------------------------------ step 0

def widen(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen logits exactly to float64.  bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        bits32 = np.asarray(logits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(logits, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------------ step 1

def softmax(rows: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(rows / T) along the last axis, in float64.

    The row maximum is subtracted before exponentiating; this changes nothing
    mathematically and keeps exp in range.
    """
    if not temperature > 0.0:
        raise ValueError("softmax needs T > 0")
    m = rows.max(axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("row with no finite logit (all -inf, +inf or NaN)")
    e = np.exp((rows - m) / temperature)
    return e / e.sum(axis=-1, keepdims=True)


def argmax_first(rows: np.ndarray) -> np.ndarray:
    """Index of the row maximum, lowest index on ties (-0.0 equals +0.0)."""
    return np.argmax(rows, axis=-1)


# ------------------------------------------------------------------ step 2

def overlap(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """alpha = sum_x min(p(x), q(x))."""
    return np.minimum(p, q).sum(axis=-1)


def total_variation(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """TV(p, q) = 1/2 sum_x |p(x) - q(x)|."""
    return 0.5 * np.abs(p - q).sum(axis=-1)


# ------------------------------------------------------------------ step 3

def ratio_test(p_x: np.ndarray, q_x: np.ndarray, u: np.ndarray, lenience: float = 1.0):
    """Accept iff u <= min(1, p(x) / (l q(x))).  Returns (accept, min(1, ratio))."""
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = p_x / (lenience * q_x)
    capped = np.minimum(1.0, ratio)          # NaN propagates, so 0/0 rejects
    return u <= capped, capped


def accepted_prefix(accept: np.ndarray) -> np.ndarray:
    """n = index of the first rejection along the last axis, or its length."""
    gamma = accept.shape[-1]
    if gamma == 0:
        return np.zeros(accept.shape[:-1], dtype=np.int64)
    rejected = ~accept
    return np.where(rejected.any(axis=-1), np.argmax(rejected, axis=-1), gamma)


# ------------------------------------------------------------------ step 4

def residual_weights(p_row: np.ndarray, q_row: np.ndarray, lenience: float = 1.0) -> np.ndarray:
    """max(0, p - l q), not yet normalised (l = 1: the exact residual)."""
    return np.maximum(0.0, p_row - lenience * q_row)


# ------------------------------------------------------------------ step 5

def inverse_cdf(probs: np.ndarray, u: np.ndarray):
    """First token whose cumulative probability exceeds u (token-index order).

    probs: [N, V] normalised weights; u: [N].  If rounding leaves every
    cumulative sum <= u, the last token with positive weight is taken.
    Returns (token [N], cdf [N, V]).
    """
    cdf = np.cumsum(probs, axis=-1)
    above = cdf > u[:, None]
    token = np.argmax(above, axis=-1)
    none = ~above.any(axis=-1)
    if none.any():
        V = probs.shape[-1]
        last_pos = V - 1 - np.argmax(probs[:, ::-1] > 0, axis=-1)
        token = np.where(none, last_pos, token)
    return token, cdf


# ------------------------------------------------- decision margins
#
# How close each discrete decision came to going the other way, for comparing
# with results computed in other arithmetic.  They change no result.

def in_u_band(u: np.ndarray, capped: np.ndarray) -> np.ndarray:
    """Accept tests whose uniform lies within U_BAND of min(1, ratio)."""
    with np.errstate(invalid="ignore"):
        return np.abs(u - capped) < U_BAND


def cdf_margin(cdf: np.ndarray, u: np.ndarray) -> np.ndarray:
    """min_j |cdf_j - u| per row: the distance of the uniform from the nearest
    step of the sampled row's normalised cumulative weights."""
    return np.abs(cdf - u[:, None]).min(axis=-1)


# ------------------------------------------------------------ whole step

@dataclasses.dataclass
class Result:
    n_accepted: np.ndarray      # int64 [B]
    next_token: np.ndarray      # int64 [B]
    alpha: np.ndarray           # float64 [B, gamma]
    tv: np.ndarray              # float64 [B, gamma]
    p_draft: np.ndarray         # float64 [B, gamma]  p_i(x_i)
    q_draft: np.ndarray         # float64 [B, gamma]  q_i(x_i)
    u_band: np.ndarray          # bool [B]: an evaluated accept test lies within U_BAND
    cdf_margin: np.ndarray      # float64 [B]: min_j |u_gamma - cdf_j| of the sampled row
    residual: np.ndarray        # bool [B]: sampled from a residual (else bonus / argmax)
    weights: np.ndarray | None  # float64 [B, V] normalised sampling row, if requested
    filter_margin: np.ndarray | None = None  # float64 [B]: smallest top-p margin of the sequence's rows
    res_mass: np.ndarray | None = None  # float64 [B]: mass of the residual after a rejection, else NaN
    # per row (target rows 0..gamma, then draft rows 0..gamma-1) with top-k /
    # top-p: the keep threshold and the nucleus margin; None without filters
    filter_tau: np.ndarray | None = None      # float64 [B, 2 gamma + 1]
    filter_margins: np.ndarray | None = None  # float64 [B, 2 gamma + 1]


def _verify_block(target, draft, tokens, u, temperature, dtype, keep_weights, lenience=1.0, gseq=None,
                  top_k=0, top_p=1.0):
    tl = widen(target, dtype)            # [b, gamma+1, V]
    dl = widen(draft, dtype)             # [b, gamma, V]
    nb, g1, V = tl.shape
    gamma = g1 - 1
    rows = np.arange(nb)
    tokens = np.asarray(tokens, dtype=np.int64).reshape(nb, gamma)
    # per-sequence draft counts; a position i >= gamma_b is padding
    gb = np.full(nb, gamma, dtype=np.int64) if gseq is None else np.asarray(gseq, dtype=np.int64)
    live = np.arange(gamma)[None, :] < gb[:, None]                     # [b, gamma]
    tok = np.where(live, tokens, 0)                                      # padding is never looked up
    u_final = u[rows, gb]
    if gseq is not None:
        # padding rows take no part: zero them so nothing of theirs can leak in
        tl = np.where((np.arange(g1)[None, :] <= gb[:, None])[..., None], tl, 0.0)
        dl = np.where(live[..., None], dl, 0.0)
    fmargin = np.full(nb, np.inf)
    ftau = fmg = None
    if temperature > 0.0 and ((0 < top_k < V) or top_p < 1.0):
        # top-k / top-p adjust p and q the same way before anything else
        tau_t, mg_t = adjust.thresholds(tl, temperature, top_k, top_p)
        tau_d, mg_d = adjust.thresholds(dl, temperature, top_k, top_p)
        tl, dl = adjust.apply(tl, tau_t), adjust.apply(dl, tau_d)
        fmargin = np.minimum(mg_t.min(axis=-1), mg_d.min(axis=-1) if gamma else np.inf)
        ftau = np.concatenate([tau_t, tau_d], axis=1)
        fmg = np.concatenate([mg_t, mg_d], axis=1)

    if temperature == 0.0:
        a = argmax_first(tl)             # target argmax per position
        d = argmax_first(dl)             # draft argmax per position
        alpha = np.where(live, (a[:, :gamma] == d).astype(np.float64), np.nan)
        p_x = np.where(live, (tok == a[:, :gamma]).astype(np.float64), np.nan)
        q_x = np.where(live, (tok == d).astype(np.float64), np.nan)
        accept = (tok == a[:, :gamma]) & live
        n = accepted_prefix(accept)      # at most gamma_b: the first padding position stops it
        t = a[rows, n]
        weights = None
        if keep_weights:
            weights = np.zeros((nb, V))
            weights[rows, t] = 1.0
        return Result(n, t, alpha, 1.0 - alpha, p_x, q_x, np.zeros(nb, bool),
                      np.full(nb, np.inf), np.zeros(nb, bool), weights, fmargin, np.full(nb, np.nan),
                      ftau, fmg)

    p = softmax(tl, temperature)         # [b, gamma+1, V]
    q = softmax(dl, temperature)         # [b, gamma, V]
    alpha = np.where(live, overlap(p[:, :gamma], q), np.nan)
    tv = np.where(live, total_variation(p[:, :gamma], q), np.nan)
    p_x = np.take_along_axis(p[:, :gamma], tok[..., None], axis=-1)[..., 0]
    q_x = np.take_along_axis(q, tok[..., None], axis=-1)[..., 0]
    accept, capped = ratio_test(p_x, q_x, u[:, :gamma], lenience)
    accept &= live
    n = accepted_prefix(accept)          # at most gamma_b: the first padding position stops it
    p_x = np.where(live, p_x, np.nan)
    q_x = np.where(live, q_x, np.nan)

    evaluated = (np.arange(gamma)[None, :] <= n[:, None]) & live
    near = in_u_band(u[:, :gamma], capped)
    u_band = (near & evaluated).any(axis=-1) if gamma else np.zeros(nb, bool)

    residual = n < gb
    w = p[rows, n].copy()                          # bonus row p_{gamma_b} when n == gamma_b
    res_mass = np.full(nb, np.nan)
    if residual.any():
        idx = np.nonzero(residual)[0]
        res = residual_weights(p[idx, n[idx]], q[idx, n[idx]], lenience)
        mass = res.sum(axis=-1)
        res_mass[idx] = mass
        ok = mass > 0.0                            # no mass at all: keep p_n
        w[idx[ok]] = res[ok] / mass[ok][:, None]
    w /= w.sum(axis=-1, keepdims=True)
    t, cdf = inverse_cdf(w, u_final.astype(np.float64))
    margin = cdf_margin(cdf, u_final)
    return Result(n, t, alpha, tv, p_x, q_x, u_band, margin, residual,
                  w if keep_weights else None, fmargin, res_mass, ftau, fmg)


def verify(target, draft, tokens, uniforms, temperature: float, dtype: str,
           keep_weights: bool = False, block_elems: int = 1 << 25, lenience: float = 1.0,
           gamma_seq=None, top_k: int = 0, top_p: float = 1.0, workers: int = 1) -> Result:
    """Run the verification step for every sequence of the batch.

    target [B, gamma+1, V], draft [B, gamma, V] (float32, or uint16 bf16 bits),
    tokens int [B, gamma], uniforms float32 [B, gamma+1] in (0, 1).
    lenience l in (0, 1] and gamma_seq int [B] with 0 <= gamma_b <= gamma are the
    two extensions described in the module notes; top_k and top_p adjust every
    row first (oracle/adjust.py; top_k <= 0 and top_p >= 1 disable them).
    temperature, lenience and top_p are taken as the 32-bit floats a caller of
    the library passes.
    Sequences are independent, so they are processed in blocks to bound memory,
    on `workers` threads (NumPy releases the interpreter lock in its loops); the
    blocks are computed exactly as on one thread.
    """
    target = np.asarray(target)
    draft = np.asarray(draft)
    B, g1, V = target.shape
    gamma = g1 - 1
    if draft.shape != (B, gamma, V):
        raise ValueError("draft must be [B, gamma, V]")
    if temperature < 0.0 or not np.isfinite(temperature):
        raise ValueError("temperature must be finite and >= 0")
    if not (0.0 < lenience <= 1.0):
        raise ValueError("lenience must be in (0, 1]")
    if not (top_p > 0.0):
        raise ValueError("top_p must be > 0")
    if gamma_seq is not None:
        gamma_seq = np.asarray(gamma_seq, dtype=np.int64).reshape(B)
        if (gamma_seq < 0).any() or (gamma_seq > gamma).any():
            raise ValueError("every gamma_b must lie in [0, gamma]")
    u = np.asarray(uniforms, dtype=np.float32).astype(np.float64).reshape(B, g1)
    tokens = np.asarray(tokens).reshape(B, gamma)
    temperature, lenience, top_p = (float(np.float32(v)) for v in (temperature, lenience, top_p))
    per_seq = max(1, (2 * gamma + 1) * V)
    step = max(1, block_elems // per_seq)
    if workers > 1:
        step = min(step, -(-B // workers))       # at least one block per worker

    def block(s):
        return _verify_block(target[s:s + step], draft[s:s + step], tokens[s:s + step],
                             u[s:s + step], temperature, dtype, keep_weights, lenience,
                             None if gamma_seq is None else gamma_seq[s:s + step], top_k, top_p)

    starts = range(0, B, step)
    if workers > 1 and len(starts) > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(block, starts))
    else:
        parts = [block(s) for s in starts]
    if not parts:
        z = np.zeros(0)
        return Result(z.astype(np.int64), z.astype(np.int64), np.zeros((0, gamma)),
                      np.zeros((0, gamma)), np.zeros((0, gamma)), np.zeros((0, gamma)),
                      z.astype(bool), z, z.astype(bool), None, z, z)
    cat = lambda f: np.concatenate([getattr(r, f) for r in parts])  # noqa: E731
    filtered = parts[0].filter_tau is not None
    return Result(cat("n_accepted"), cat("next_token"), cat("alpha"), cat("tv"),
                  cat("p_draft"), cat("q_draft"), cat("u_band"), cat("cdf_margin"),
                  cat("residual"), cat("weights") if keep_weights else None, cat("filter_margin"),
                  cat("res_mass"), cat("filter_tau") if filtered else None,
                  cat("filter_margins") if filtered else None)


def verify_case(case, keep_weights: bool = False, seqs=None, lenience: float = 1.0, gamma_seq=None,
                top_k: int = 0, top_p: float = 1.0, workers: int = 1) -> Result:
    """verify() on a workloads.VerifyCase, optionally on a subset of sequences."""
    if seqs is not None:
        case = case.subset(seqs)
        if gamma_seq is not None:
            gamma_seq = np.asarray(gamma_seq)[np.asarray(seqs)]
    return verify(case.target, case.draft, case.tokens, case.uniforms,
                  case.temperature, case.dtype, keep_weights, lenience=lenience, gamma_seq=gamma_seq,
                  top_k=top_k, top_p=top_p, workers=workers)
