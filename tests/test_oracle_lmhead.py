"""The fp64 LM-head product against integer arithmetic and a brute-force loop."""

import numpy as np

import workloads as W
from oracle import lmhead


def test_integer_inputs_are_exact():
    # small integers are exact in bf16, so the product is an exact integer
    rng = np.random.default_rng(0)
    h = rng.integers(-8, 9, size=(5, 37))
    w = rng.integers(-8, 9, size=(37, 29))
    got = lmhead.logits(W.f32_to_bf16_bits(h.astype(np.float32)), W.f32_to_bf16_bits(w.astype(np.float32)))
    want = [[sum(int(h[m, k]) * int(w[k, v]) for k in range(37)) for v in range(29)] for m in range(5)]
    assert np.array_equal(got, np.array(want, dtype=np.float64))


def test_brute_force_and_column_window():
    rng = np.random.default_rng(1)
    hb = W.f32_to_bf16_bits(rng.standard_normal((3, 16)).astype(np.float32))
    wb = W.f32_to_bf16_bits(rng.standard_normal((16, 40)).astype(np.float32) * 0.1)
    hf, wf = W.bf16_bits_to_f32(hb).astype(np.float64), W.bf16_bits_to_f32(wb).astype(np.float64)
    full = lmhead.logits(hb, wb, col_block=7)
    for m in range(3):
        for v in range(40):
            s = 0.0
            for k in range(16):
                s += hf[m, k] * wf[k, v]
            assert abs(full[m, v] - s) < 1e-12
    part = lmhead.logits(hb, wb, cols=slice(11, 30), col_block=5)
    assert np.array_equal(part, full[:, 11:30])
    bound = lmhead.abs_error_bound(hb, wb)
    assert bound.shape == full.shape and np.all(bound > 0)
