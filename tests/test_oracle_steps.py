"""Step-level pins of the fp64 oracle: each step against a library routine, a
brute-force loop, a closed form or a value the pages print."""

import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
    EX = json.load(f)


def _probs(xs):
    from fractions import Fraction as F
    return np.array([float(F(x)) for x in xs])


def _logits(p):
    with np.errstate(divide="ignore"):
        return np.log(p)


# ------------------------------------------------------------- widening

def test_widen_bf16_exact():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x7F80, 0xFF80, 0x0001], np.uint16)
    got = ov.widen(bits, "bf16")
    want = [0.0, -0.0, 1.0, -1.0, 3.140625, np.inf, -np.inf, 2.0 ** -133]
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[1])


def test_widen_f32_exact():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(ov.widen(x, "f32"), x.astype(np.float64))


# -------------------------------------------------------------- softmax

@pytest.mark.parametrize("T", [0.05, 0.7, 1.0, 3.0])
def test_softmax_matches_scipy(T):
    x = np.random.default_rng(1).standard_normal((7, 513)) * 4
    np.testing.assert_allclose(ov.softmax(x, T), scipy.special.softmax(x / T, axis=-1), rtol=1e-12, atol=1e-300)


def test_softmax_constant_row_and_shift_invariance():
    V = 1000
    np.testing.assert_allclose(ov.softmax(np.full((1, V), 3.5), 1.0), 1.0 / V, rtol=1e-14)
    x = np.random.default_rng(2).standard_normal((3, 200)) * 3
    for shift in (-700.0, 0.25, 900.0):
        np.testing.assert_allclose(ov.softmax(x + shift, 0.9), ov.softmax(x, 0.9), rtol=1e-9, atol=1e-300)


def test_softmax_neg_inf_entries_get_zero_and_bad_rows_raise():
    x = np.array([[0.0, -np.inf, 1.0, -np.inf]])
    p = ov.softmax(x, 1.0)
    assert p[0, 1] == 0 and p[0, 3] == 0
    np.testing.assert_allclose(p[0, [0, 2]], scipy.special.softmax([0.0, 1.0]), rtol=1e-15)
    with pytest.raises(ValueError):
        ov.softmax(np.full((1, 4), -np.inf), 1.0)
    with pytest.raises(ValueError):
        ov.softmax(x, 0.0)


def test_softmax_temperature_tends_to_argmax():
    x = np.array([[0.3, 2.0, 1.9, -5.0]])
    p = ov.softmax(x, 0.001)
    assert p[0, 1] == 1.0 and p[0, 2] < 1e-40 and p[0].sum() == 1.0


# --------------------------------------------------------------- argmax

def test_argmax_first_matches_brute_force_with_ties():
    rng = np.random.default_rng(3)
    for _ in range(300):
        V = int(rng.integers(1, 12))
        row = rng.integers(-3, 3, size=V).astype(np.float64)
        best = 0
        for j in range(1, V):
            if row[j] > row[best]:
                best = j
        assert ov.argmax_first(row[None])[0] == best


def test_argmax_signed_zero_is_a_tie():
    assert ov.argmax_first(np.array([[-0.0, 0.0, -1.0]]))[0] == 0
    assert ov.argmax_first(np.array([[-1.0, -0.0, 0.0]]))[0] == 1


# ------------------------------------------------------- overlap and TV

@pytest.mark.parametrize("name", ["W3", "W4", "W100"])
def test_overlap_worked_examples_through_softmax(name):
    ex = EX[name]
    p = ov.softmax(_logits(_probs(ex["p"]))[None], 1.0)
    q = ov.softmax(_logits(_probs(ex["q"]))[None], 1.0)
    from fractions import Fraction as F
    assert ov.overlap(p, q)[0] == pytest.approx(float(F(ex["alpha"])), abs=1e-15)


def test_overlap_identity_and_bounds_random():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 300)) * 3
    y = x + rng.standard_normal((50, 300))
    p, q = ov.softmax(x, 1.0), ov.softmax(y, 1.0)
    a = ov.overlap(p, q)
    np.testing.assert_allclose(a, 1.0 - ov.total_variation(p, q), atol=1e-14)
    assert np.all(a >= 0) and np.all(a <= 1)
    # plain rejection sampling accepts 1/r_max of the time, never more than alpha
    assert np.all(1.0 / (p / q).max(axis=-1) <= a + 1e-15)
    np.testing.assert_allclose(ov.overlap(p, p), 1.0, atol=1e-14)


# ----------------------------------------------------------- ratio test

def test_ratio_test_ieee_semantics():
    p_x = np.array([0.3, 0.5, 0.2, 0.0, 0.7, 0.0])
    q_x = np.array([0.5, 0.5, 0.0, 0.0, 0.1, 0.4])
    u = np.array([0.6, 0.999, 0.999, 0.5, 0.999, 1e-7])
    acc, capped = ov.ratio_test(p_x, q_x, u)
    # 0.6 <= 0.6 accepts (<=); ratio 1; q=0<p gives +inf -> accept; 0/0 -> NaN -> reject;
    # ratio 7 capped at 1; p = 0 rejects for any u > 0
    assert acc.tolist() == [True, True, True, False, True, False]
    assert capped[0] == pytest.approx(0.6) and capped[4] == 1.0 and np.isnan(capped[3])


def test_accepted_prefix_brute_force():
    rng = np.random.default_rng(5)
    acc = rng.random((500, 6)) < 0.7
    n = ov.accepted_prefix(acc)
    for r in range(500):
        k = 0
        while k < 6 and acc[r, k]:
            k += 1
        assert n[r] == k
    assert ov.accepted_prefix(np.zeros((3, 0), bool)).tolist() == [0, 0, 0]


# ------------------------------------------------------------- residual

@pytest.mark.parametrize("name", ["W3", "W4", "W100"])
def test_residual_worked_examples(name):
    ex = EX[name]
    p, q = _probs(ex["p"]), _probs(ex["q"])
    w = ov.residual_weights(p, q)
    if "residual_mass" in ex:
        np.testing.assert_allclose(w, _probs(ex["residual_mass"]), atol=1e-15)
    if "residual_distribution" in ex:
        np.testing.assert_allclose(w / w.sum(), _probs(ex["residual_distribution"]), atol=1e-15)
    # residual mass equals the rejection mass 1 - alpha
    assert w.sum() == pytest.approx(1 - ov.overlap(p, q), abs=1e-15)


# ----------------------------------------------------------- inverse CDF

def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(6)
    for _ in range(300):
        V = int(rng.integers(1, 9))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[int(rng.integers(V))] = 1.0
        w = w / w.sum()
        u = rng.random()
        acc, want = 0.0, None
        for j in range(V):
            acc += w[j]
            if acc > u:
                want = j
                break
        if want is None:
            want = max(j for j in range(V) if w[j] > 0)
        got, _ = ov.inverse_cdf(w[None], np.array([u]))
        assert got[0] == want
        assert w[got[0]] > 0
        assert got[0] == np.searchsorted(np.cumsum(w), u, side="right") or want == max(
            j for j in range(V) if w[j] > 0)


def test_inverse_cdf_strict_boundary_and_guard():
    w = np.array([[0.5, 0.0, 0.5]])
    assert ov.inverse_cdf(w, np.array([0.5]))[0][0] == 2     # strict ">" skips token 0 at its edge
    assert ov.inverse_cdf(w, np.array([0.49]))[0][0] == 0
    # rounding guard: u above every cumulative value -> last positive-weight token
    w = np.array([[0.25, 0.25, 0.25, 0.0]])
    assert ov.inverse_cdf(w, np.array([0.9]))[0][0] == 2


# ------------------------------------------------ small residual masses

@pytest.mark.parametrize("delta", [2.0 ** -8, 2.0 ** -16, 2.0 ** -21])
def test_small_residual_mass_is_sampled(delta):
    """Two tokens: target logits (delta, 0), draft logits (0, 0), so p(0) =
    1/(1 + e^-delta), about 1/2 + delta/4, and q = (1/2, 1/2).  Draft x = 1 has
    ratio 1 - 2 (p(0) - 1/2), below the largest uniform 1 - 2^-24, so it is
    rejected.  The residual max(0, p - q) sits on token 0 alone, with mass
    about delta/4 (2^-23 at the smallest delta), and [FI] eq. (2) samples it
    after any rejection: the token is 0 whatever the final uniform is."""
    target = np.array([[[delta, 0.0], [0.0, 0.0]]], np.float32)
    draft = np.zeros((1, 1, 2), np.float32)
    for u_final in (0.01, 0.9, 1.0 - 2.0 ** -24):
        u = np.array([[1.0 - 2.0 ** -24, u_final]], np.float32)
        res = ov.verify(target, draft, np.array([[1]]), u, 1.0, "f32")
        assert res.n_accepted[0] == 0
        mass = 1.0 / (1.0 + np.exp(-np.float64(np.float32(delta)))) - 0.5
        np.testing.assert_allclose(res.res_mass[0], mass, rtol=1e-6)
        assert res.next_token[0] == 0


def test_zero_residual_mass_samples_p():
    """Identical rows and a draft token with p(x) = q(x) = 0 (logit -inf in both):
    0/0 rejects, the residual has no mass, and the token is drawn from p_0
    itself ([LH] "Three candidates explain the acceptance rule": a zero-mass
    residual is not normalised)."""
    row = np.array([0.0, 1.0, -np.inf, 0.5], np.float32)
    target = np.stack([row, row])[None]
    draft = row[None, None].copy()
    p = np.exp(row.astype(np.float64) - 1.0)
    p /= p.sum()
    for u_final, want in ((0.01, 0), (p[0] + 0.01, 1), (p[0] + p[1] + 0.01, 3)):
        u = np.array([[0.5, u_final]], np.float32)
        res = ov.verify(target, draft, np.array([[2]]), u, 1.0, "f32")
        assert res.n_accepted[0] == 0 and res.res_mass[0] == 0.0
        assert res.next_token[0] == want


@pytest.mark.parametrize("L", [-20.0, -45.0, -70.0])
def test_tiny_residual_mass_is_sampled(L):
    """Target logits (0, 0, -inf) give p = (1/2, 1/2, 0); draft logits (0, 0, L)
    put q(2) = e^L / (2 + e^L) on the token the target excludes.  Drafting x = 2
    is always rejected (p(x) = 0), and the residual is (q(2)/2, q(2)/2, 0): a
    mass of about e^L (down to 1e-31 here), split evenly, which is sampled
    like any other residual -- u below 1/2 gives token 0, above gives token 1,
    never token 2 ([FI] eq. (2)).  In fp64 each p - q cancels to within an
    ulp of 1/2, so the mass is checked to that absolute accuracy (below it the
    fp64 residual is exactly zero and the fall-back p_0 is the same
    distribution)."""
    target = np.array([[[0.0, 0.0, -np.inf], [0.0, 0.0, -np.inf]]], np.float32)
    draft = np.array([[[0.0, 0.0, L]]], np.float32)
    q2 = np.exp(np.float64(np.float32(L))) / (2.0 + np.exp(np.float64(np.float32(L))))
    for u_final, want in ((0.25, 0), (0.75, 1), (0.5 - 2.0 ** -20, 0), (0.5 + 2.0 ** -20, 1)):
        u = np.array([[0.3, u_final]], np.float32)
        res = ov.verify(target, draft, np.array([[2]]), u, 1.0, "f32")
        assert res.n_accepted[0] == 0
        np.testing.assert_allclose(res.res_mass[0], q2, rtol=1e-12, atol=2.0 ** -53)
        assert res.next_token[0] == want
