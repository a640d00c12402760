"""Pins of the oracle's decision margins: the flags and distances that decide
which rows the GPU comparison may exempt (tests/parity.py).

Each margin is placed at a known distance from its decision boundary on a tiny
input whose probabilities are known in closed form:

  * the u band: the accept uniform at min(1, p/q) +- 5e-7 (inside the 1e-6
    band) and +- 2e-6 (outside), and a band position after the first
    rejection, which is never evaluated and so never flagged;
  * the CDF margin: the final uniform a known distance from a step of the
    bonus row's CDF, exactly on a step (strict ">" takes the next token), and
    on the normalised residual of [FI]'s 4-token example;
  * the nucleus margin: top_p a known distance above and below a cumulative
    mass of a row with exact probabilities.

Planted mistakes (a band of 1, margins forced to 0 or to infinity) must fail
these pins.
"""

import numpy as np
import pytest

from oracle import adjust
from oracle import verify as ov


def _f32(x):
    return float(np.float32(x))


# ----------------------------------------------------------------- u band

def _two_token_ratio():
    """Target logits (-1, 0), draft logits (0, 0): q = (1/2, 1/2) and
    p(0) = 1 / (1 + e), so drafting token 0 has ratio r = 2 / (1 + e)."""
    target = np.array([[[-1.0, 0.0], [0.0, 0.0]]], np.float32)
    draft = np.zeros((1, 1, 2), np.float32)
    r = 2.0 / (1.0 + np.e)
    return target, draft, r


@pytest.mark.parametrize("d,flagged", [(5e-7, True), (-5e-7, True), (2e-6, False), (-2e-6, False),
                                       (9e-7, True), (-1.1e-6, False)])
def test_u_band_flag_at_known_distance(d, flagged):
    target, draft, r = _two_token_ratio()
    u0 = _f32(r + d)
    assert abs(abs(u0 - r) - abs(d)) < 6e-8          # fp32 spacing near 0.54 is 6e-8
    u = np.array([[u0, 0.5]], np.float32)
    res = ov.verify(target, draft, np.array([[0]]), u, 1.0, "f32")
    assert res.n_accepted[0] == (1 if u0 <= r else 0)
    assert bool(res.u_band[0]) is flagged
    np.testing.assert_allclose(res.p_draft[0, 0] / res.q_draft[0, 0], r, rtol=1e-14)


def test_u_band_ignores_positions_after_the_first_rejection():
    """Position 0 rejects clearly (u = 0.99 against r = 0.54); position 1's
    uniform sits on its ratio but is never evaluated."""
    _, _, r = _two_token_ratio()
    target = np.array([[[-1.0, 0.0], [-1.0, 0.0], [0.0, 0.0]]], np.float32)
    draft = np.zeros((1, 2, 2), np.float32)
    u = np.array([[0.99, _f32(r), 0.5]], np.float32)
    res = ov.verify(target, draft, np.array([[0, 0]]), u, 1.0, "f32")
    assert res.n_accepted[0] == 0
    assert not res.u_band[0]
    u[0, 0] = _f32(r - 1e-7)                          # now position 0 is in the band too
    res = ov.verify(target, draft, np.array([[0, 0]]), u, 1.0, "f32")
    assert res.u_band[0]


def test_u_band_at_ratio_above_one_uses_the_cap():
    """Drafting token 1 (p = e/(1+e) > q = 1/2) caps the ratio at 1, so only a
    uniform within 1e-6 of 1 is in the band."""
    target, draft, _ = _two_token_ratio()
    for u0, flagged in ((1.0 - 2.0 ** -24, True), (1.0 - 2e-6, False), (0.5, False)):
        res = ov.verify(target, draft, np.array([[1]]), np.array([[u0, 0.5]], np.float32), 1.0, "f32")
        assert res.n_accepted[0] == 1
        assert bool(res.u_band[0]) is flagged


# ------------------------------------------------------------ CDF margin

def _bonus_case(u_final):
    """gamma = 1, the draft accepted with certainty (p = q, u small); the bonus
    row p_1 = (1/4, 1/2, 1/4) from logits (0, ln 2, 0): steps at 1/4, 3/4, 1."""
    row1 = np.array([0.0, np.log(2.0), 0.0], np.float32)
    row0 = np.array([0.0, 0.0, 0.0], np.float32)
    target = np.stack([row0, row1])[None]
    draft = row0[None, None].copy()
    u = np.array([[0.5, u_final]], np.float32)
    res = ov.verify(target, draft, np.array([[0]]), u, 1.0, "f32", keep_weights=True)
    assert res.n_accepted[0] == 1
    return res


@pytest.mark.parametrize("d", [3e-6, -3e-6, 2e-5, -4e-7])
def test_cdf_margin_at_known_distance_from_a_step(d):
    u0 = _f32(0.25 + d)
    res = _bonus_case(u0)
    w = res.weights[0]
    np.testing.assert_allclose(np.cumsum(w), [0.25, 0.75, 1.0], atol=1e-7)  # ln 2 rounded to fp32
    step = np.cumsum(w)[0]
    np.testing.assert_allclose(res.cdf_margin[0], abs(u0 - step), rtol=1e-9, atol=1e-15)
    assert res.next_token[0] == (0 if u0 < step else 1)


def test_cdf_margin_zero_on_a_step_takes_the_next_token():
    # a row whose first step is exactly representable: p_1 = (1/2, 1/2)
    target = np.zeros((1, 2, 2), np.float32)
    draft = np.zeros((1, 1, 2), np.float32)
    res = ov.verify(target, draft, np.array([[0]]), np.array([[0.5, 0.5]], np.float32), 1.0, "f32")
    assert res.n_accepted[0] == 1
    assert res.cdf_margin[0] == 0.0
    assert res.next_token[0] == 1                      # strict ">": token 0 needs cdf > 0.5


def test_cdf_margin_of_a_residual_row_is_normalised():
    """[FI]'s 4-token example: p = (.5, .3, .15, .05), q = (.3, .5, .1, .1); the
    residual normalises to (.8, 0, .2, 0), steps at .8, .8, 1, 1."""
    p = np.array([0.5, 0.3, 0.15, 0.05])
    q = np.array([0.3, 0.5, 0.1, 0.1])
    target = np.stack([np.log(p), np.log(p)]).astype(np.float32)[None]
    draft = np.log(q).astype(np.float32)[None, None]
    for d in (1e-5, -1e-5, 2e-6):
        u0 = _f32(0.8 + d)
        u = np.array([[0.9, u0]], np.float32)           # 0.9 > p/q = 0.6: token 1 rejected
        res = ov.verify(target, draft, np.array([[1]]), u, 1.0, "f32", keep_weights=True)
        assert res.n_accepted[0] == 0 and res.residual[0]
        step = res.weights[0][0]
        np.testing.assert_allclose(step, 0.8, atol=1e-7)
        np.testing.assert_allclose(res.cdf_margin[0], abs(u0 - step), rtol=1e-9, atol=1e-15)
        assert res.next_token[0] == (0 if u0 < step else 2)


# --------------------------------------------------------- nucleus margin

P4 = np.array([0.5, 0.3, 0.15, 0.05])


@pytest.mark.parametrize("top_p,keep,margin", [
    (0.8 + 1e-4, 3, 1e-4),          # just past the second step: the third group joins
    (0.8 - 3e-5, 2, 3e-5),          # just short of it: two groups suffice
    (0.95, 3, 0.0),                 # exactly a step (in fp64): >= keeps three
    (0.3, 1, 0.2),                  # inside the first group
    (0.9, 3, 0.05),
])
def test_nucleus_margin_at_known_distance(top_p, keep, margin):
    row = np.log(P4)
    tau, mg = adjust.topp_threshold(row, 1.0, top_p)
    assert int((row >= tau).sum()) == keep
    np.testing.assert_allclose(mg, margin, atol=1e-12)


def test_nucleus_margin_is_over_the_top_k_survivors():
    """After top-k 2 the survivors renormalise to (5/8, 3/8): top_p 0.6 lies
    0.025 below the first step."""
    row = np.log(P4)
    tk = adjust.topk_threshold(row, 2)
    tau, mg = adjust.topp_threshold(row, 1.0, 0.6, tk)
    assert int((row >= tau).sum()) == 1
    np.testing.assert_allclose(mg, 0.025, atol=1e-12)


def test_filter_margin_reaches_the_result():
    """verify() reports the smallest nucleus margin among a sequence's rows."""
    row = np.log(P4).astype(np.float32)
    target = np.stack([row, row])[None]
    draft = row[None, None].copy()
    res = ov.verify(target, draft, np.array([[0]]), np.array([[0.5, 0.5]], np.float32), 1.0, "f32",
                    top_p=0.8 + 1e-4)
    # top_p reaches the oracle as the 32-bit float the library would receive;
    # the logits are log(P4) rounded to fp32, so the step is 0.8 to about 1e-8
    p = np.exp(row.astype(np.float64))
    p /= p.sum()
    np.testing.assert_allclose(res.filter_margin[0], abs(_f32(0.8 + 1e-4) - (p[0] + p[1])), rtol=1e-9)


# -------------------------------------------------------- planted mistakes

def _run_all():
    for d, f in ((5e-7, True), (-2e-6, False)):
        test_u_band_flag_at_known_distance(d, f)
    test_u_band_ignores_positions_after_the_first_rejection()
    for d in (3e-6, -3e-6):
        test_cdf_margin_at_known_distance_from_a_step(d)
    test_cdf_margin_of_a_residual_row_is_normalised()
    test_nucleus_margin_at_known_distance(0.8 + 1e-4, 3, 1e-4)
    test_filter_margin_reaches_the_result()


@pytest.mark.parametrize("mutant", ["u_band_one", "u_band_zero", "cdf_margin_zero", "cdf_margin_inf",
                                    "nucleus_margin_zero", "nucleus_margin_inf", "u_band_all_positions"])
def test_planted_mistakes_in_the_margins_are_caught(mutant, monkeypatch):
    if mutant == "u_band_one":
        monkeypatch.setattr(ov, "U_BAND", 1.0)
    elif mutant == "u_band_zero":
        monkeypatch.setattr(ov, "U_BAND", 0.0)
    elif mutant == "cdf_margin_zero":
        monkeypatch.setattr(ov, "cdf_margin", lambda cdf, u: np.zeros(cdf.shape[0]))
    elif mutant == "cdf_margin_inf":
        monkeypatch.setattr(ov, "cdf_margin", lambda cdf, u: np.full(cdf.shape[0], np.inf))
    elif mutant == "u_band_all_positions":
        orig = ov.in_u_band
        monkeypatch.setattr(ov, "in_u_band", lambda u, c: orig(u, c) | (np.abs(u - c) < 0.5))
    else:
        orig = adjust.topp_threshold
        val = 0.0 if mutant == "nucleus_margin_zero" else np.inf
        monkeypatch.setattr(adjust, "topp_threshold", lambda *a, **k: (orig(*a, **k)[0], val))
    with pytest.raises(AssertionError):
        _run_all()


# ------------------------------------------------ in-band threshold choices

def test_adjacent_values_are_one_tie_group_either_side():
    """A row within the nucleus band may keep one tie group more or less than
    the oracle: the allowed thresholds are the oracle's and the next distinct
    finite logit on either side, never a logit two groups away."""
    from tests import parity
    x = np.array([1.0, 3.0, 2.0, 2.0, -np.inf, 5.0, 3.0])
    np.testing.assert_array_equal(parity.adjacent_values(x, 2.0), np.float32([1, 2, 3]))
    np.testing.assert_array_equal(parity.adjacent_values(x, 1.0), np.float32([1, 2]))
    np.testing.assert_array_equal(parity.adjacent_values(x, 5.0), np.float32([3, 5]))
    assert 5.0 not in parity.adjacent_values(x, 2.0)
    assert 1.0 not in parity.adjacent_values(x, 3.0)
