"""GPU parity of the LM-head product and of the fused LM-head + verify path,
through the C ABI, against the fp64 oracle."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import lmhead as olm
from tests import gpu_util, parity

pytestmark = pytest.mark.gpu


def _sv():
    import speculative_sampling_verification_02_amd as sv
    return sv


@pytest.fixture(scope="module")
def dev():
    return gpu_util.device()


def _bf16(arr, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)


# Shapes spanning 1..5 row tiles (several passes past 64 rows), hidden sizes of
# one and many steps, and vocabularies with a ragged last workgroup and slab.
SHAPES = [(1, 32, 8), (5, 64, 136), (16, 96, 1000), (40, 256, 2056), (64, 128, 4104),
          (65, 64, 520), (130, 32, 1032), (33, 4096, 1544)]


@pytest.mark.parametrize("M,d,V", SHAPES, ids=lambda x: str(x))
def test_integer_product_is_exact(dev, M, d, V):
    """Small integers are exact in bf16 and their fp32 sums are exact, so the
    product must equal the integer result bit for bit (this pins the matrix-core
    operand layout and every index of the kernel)."""
    rng = np.random.default_rng(M * 7919 + d * 31 + V)
    h = rng.integers(-3, 4, size=(M, d)).astype(np.float32)
    w = rng.integers(-3, 4, size=(d, V)).astype(np.float32)
    hb, wb = W.f32_to_bf16_bits(h), W.f32_to_bf16_bits(w)
    print(f"[lmhead] integer M={M} d={d} V={V}", flush=True)
    got = _sv().lmhead_logits(_bf16(hb, dev), _bf16(wb, dev)).cpu().numpy()
    want = h.astype(np.int64) @ w.astype(np.int64)
    assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("M,d,V", [(40, 4096, 8200), (7, 512, 1000)])
def test_gaussian_product_within_rounding_bound(dev, M, d, V):
    rng = np.random.default_rng(M + d + V)
    hb = W.f32_to_bf16_bits(rng.standard_normal((M, d), dtype=np.float32))
    wb = W.f32_to_bf16_bits(rng.standard_normal((d, V), dtype=np.float32) * np.float32(0.02))
    print(f"[lmhead] gaussian M={M} d={d} V={V}", flush=True)
    got = _sv().lmhead_logits(_bf16(hb, dev), _bf16(wb, dev)).cpu().numpy().astype(np.float64)
    want = olm.logits(hb, wb)
    err = np.abs(got - want)
    assert np.all(err <= olm.abs_error_bound(hb, wb)), float(err.max())
    assert float(err.max()) <= 1e-4


@pytest.fixture(scope="module")
def cfg4():
    # the full LM-head workload: B=8, gamma=4, d=4096, V=128256
    return W.config4(3, 1.0)


@pytest.fixture(scope="module")
def cfg4_gpu(cfg4, dev):
    import torch
    sv = _sv()
    c = cfg4
    print(f"[lmhead] full LM-head workload B={c.B} gamma={c.gamma} d={c.d} V={c.V}", flush=True)
    t = dict(hidden=_bf16(c.hidden, dev), wp=_bf16(c.w_target, dev), wq=_bf16(c.w_draft, dev),
             tokens=torch.from_numpy(c.tokens).to(dev), uniforms=torch.from_numpy(c.uniforms).to(dev))
    out = sv.lmhead_verify(t["hidden"], t["wp"], t["wq"], c.B, c.gamma, t["tokens"], t["uniforms"],
                           c.temperature)
    torch.cuda.synchronize(dev)
    return t, {k: v.cpu().numpy() for k, v in out.items()}


def test_full_size_logits_every_column(cfg4, cfg4_gpu):
    """GPU fp32 logits of both heads against the fp64 product on all 128256
    columns, within 1e-4 absolute and the fp32 accumulation's rounding bound."""
    c = cfg4
    _, got = cfg4_gpu
    hq = c.hidden[c.draft_hidden_rows()]
    for name, hb, wb, logits in (("target", c.hidden, c.w_target, got["target_logits"].reshape(-1, c.V)),
                                 ("draft", hq, c.w_draft, got["draft_logits"].reshape(-1, c.V))):
        for lo in range(0, c.V, 16384):
            cols = slice(lo, min(c.V, lo + 16384))
            want = olm.logits(hb, wb, cols=cols)
            err = np.abs(logits[:, cols].astype(np.float64) - want)
            assert float(err.max()) <= 1e-4, (name, lo, float(err.max()))
            assert np.all(err <= olm.abs_error_bound(hb, wb, cols=cols)), (name, lo)
        print(f"[lmhead] {name}: every column within 1e-4 and the rounding bound", flush=True)


def test_full_size_verify_on_gpu_logits(cfg4, cfg4_gpu):
    """The verification on the GPU's own fp32 logits is held to the verify
    parity rules (the oracle runs on those same logits)."""
    c = cfg4
    _, got = cfg4_gpu
    case = W.VerifyCase(name="lmhead-logits", target=got["target_logits"], draft=got["draft_logits"], dtype="f32",
                        tokens=c.tokens, uniforms=c.uniforms, temperature=c.temperature)
    rep = parity.check(case, got, where="lmhead+verify")
    print(f"[lmhead] verify on GPU logits: {rep}", flush=True)


def test_dense_draft_hidden_matches_strided(dev, cfg4, cfg4_gpu):
    import torch
    sv = _sv()
    c = cfg4
    t, got = cfg4_gpu
    hq = t["hidden"].view(c.B, c.gamma + 1, c.d)[:, :c.gamma].contiguous().view(c.B * c.gamma, c.d)
    out = sv.lmhead_verify(t["hidden"], t["wp"], t["wq"], c.B, c.gamma, t["tokens"], t["uniforms"],
                           c.temperature, hidden_draft=hq)
    torch.cuda.synchronize(dev)
    for k in ("draft_logits", "target_logits", "n_accepted", "next_token", "alpha"):
        assert np.array_equal(out[k].cpu().numpy(), got[k]), k
