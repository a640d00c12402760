"""Pins of the oracle's two extensions: the lenience factor and per-sequence
draft counts.

Lenience l ([FI] "The acceptance rate is the overlap of p and q", the paragraph
on the lenience factor): q(x) is multiplied by l before the comparison.  The
closed form the sampler must reach is derived here from that definition, with
exact rationals and independently of the oracle's code:

    kept mass      a(x) = q(x) min(1, p(x) / (l q(x))) = min(q(x), p(x) / l)
    rejected mass  beta = 1 - sum_x a(x)
    residual       r(x) = max(0, p(x) - l q(x))            (the reading taken)
    emitted        P(x) = a(x) + beta r(x) / sum r

and the page's bound P(x) <= p(x) / l is checked on it.

Per-sequence draft counts gamma_b: with identical (p, q) at every position the
tokens per round follow equation (1) with gamma_b in place of gamma ([FI]
"Tokens per target run, equation (1)"), and a padded sequence must give what the
same sequence gives unpadded.
"""

import json
import os
from fractions import Fraction as F
from math import lcm

import numpy as np
import pytest
import scipy.stats

from oracle import exact
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
    EX = json.load(f)


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def _run(p_rows, q_rows, tokens, u, lenience=1.0, gamma_seq=None):
    target = _log(p_rows).astype(np.float32)
    draft = _log(q_rows).astype(np.float32)
    return ov.verify(target, draft, tokens, u, 1.0, "f32", lenience=lenience, gamma_seq=gamma_seq)


def lenient_closed_form(p, q, l):
    """Exact emitted distribution of one lenient step (gamma = 1), from the definition."""
    a = [min(qx, px / l) for px, qx in zip(p, q)]
    beta = 1 - sum(a)
    r = [max(F(0), px - l * qx) for px, qx in zip(p, q)]
    z = sum(r)
    return [ax + (beta * rx / z if z else F(0)) for ax, rx in zip(a, r)], a, r


@pytest.mark.parametrize("name", ["W3", "W4", "W100"])
@pytest.mark.parametrize("l", [F(1, 2), F(1, 5)])
def test_lenient_exact_enumeration(name, l):
    """gamma = 1, every drafted x weighted by q(x), both uniforms on a midpoint
    grid whose cells never straddle a decision boundary: the emitted frequencies
    are the closed form exactly (to rounding)."""
    p = [F(x) for x in EX[name]["p"]]
    q = [F(x) for x in EX[name]["q"]]
    want, a, r = lenient_closed_form(p, q, l)
    assert sum(want) == 1
    # the decision boundaries: min(1, p/(l q)) for each x, and the residual CDF
    z = sum(r)
    bounds = [min(F(1), px / (l * qx)) for px, qx in zip(p, q) if qx] + \
             [sum(r[:k + 1]) / z for k in range(len(r))]
    N = lcm(*[b.denominator for b in bounds])
    assert N <= 4000, N
    V = len(p)
    g = (np.arange(N) + 0.5) / N
    u0, u1 = np.meshgrid(g, g, indexing="ij")
    u = np.stack([u0.ravel(), u1.ravel()], axis=-1).astype(np.float64)
    M = u.shape[0]
    pf, qf = np.array([float(x) for x in p]), np.array([float(x) for x in q])
    dist = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        tokens = np.full((M, 1), x, np.int64)
        res = ov.verify(np.broadcast_to(_log(pf).astype(np.float32), (M, 2, V)),
                        np.broadcast_to(_log(qf).astype(np.float32), (M, 1, V)),
                        tokens, u.astype(np.float32), 1.0, "f32", lenience=float(l))
        emitted = np.where(res.n_accepted >= 1, x, res.next_token)
        dist += float(q[x]) * np.bincount(emitted, minlength=V) / M
    np.testing.assert_allclose(dist, [float(w) for w in want], atol=2e-6)
    # the page's bound: no token more than 1/l times as often as under p
    assert all(w <= px / l for w, px in zip(want, p))


def test_lenient_chi_squared_random():
    rng = np.random.default_rng(31)
    V, trials, l = 6, 400000, 0.3
    x = rng.standard_normal(V)
    p = np.exp(x) / np.exp(x).sum()
    y = x + rng.standard_normal(V)
    q = np.exp(y) / np.exp(y).sum()
    want, _, _ = lenient_closed_form([F(v) for v in p], [F(v) for v in q], F(l))
    want = np.array([float(w) for w in want])
    tokens = rng.choice(V, size=(trials, 1), p=q)
    u = np.clip(rng.random((trials, 2)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    res = _run(np.broadcast_to(p, (trials, 2, V)), np.broadcast_to(q, (trials, 1, V)), tokens, u, l)
    counts = np.bincount(np.where(res.n_accepted >= 1, tokens[:, 0], res.next_token), minlength=V)
    assert scipy.stats.chisquare(counts, trials * want).pvalue > 1e-4
    assert np.all(want <= p / l + 1e-12)


def test_lenience_one_is_the_exact_step_and_smaller_l_accepts_more():
    rng = np.random.default_rng(32)
    B, G, V = 64, 4, 200
    t = rng.standard_normal((B, G + 1, V)).astype(np.float32) * 2
    d = (t[:, :G] + rng.standard_normal((B, G, V)).astype(np.float32)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, G))
    u = np.clip(rng.random((B, G + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    r1 = ov.verify(t, d, tokens, u, 1.0, "f32")
    r1b = ov.verify(t, d, tokens, u, 1.0, "f32", lenience=1.0)
    for f in ("n_accepted", "next_token"):
        np.testing.assert_array_equal(getattr(r1, f), getattr(r1b, f))
    prev = r1.n_accepted
    for l in (0.7, 0.4, 0.1):
        r = ov.verify(t, d, tokens, u, 1.0, "f32", lenience=l)
        # with the same uniforms every test that passed at a larger l passes here
        assert np.all(r.n_accepted >= prev)
        # the overlap is a property of p and q, not of the test
        np.testing.assert_array_equal(r.alpha, r1.alpha)
        prev = r.n_accepted
    assert prev.sum() > r1.n_accepted.sum()
    with pytest.raises(ValueError):
        ov.verify(t, d, tokens, u, 1.0, "f32", lenience=0.0)
    with pytest.raises(ValueError):
        ov.verify(t, d, tokens, u, 1.0, "f32", lenience=1.5)


def test_lenience_leaves_argmax_mode_unchanged():
    rng = np.random.default_rng(33)
    B, G, V = 32, 5, 50
    t = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    d = (t[:, :G] + 0.5 * rng.standard_normal((B, G, V))).astype(np.float32)
    tokens = np.argmax(d, axis=-1)
    u = np.full((B, G + 1), 0.5, np.float32)
    r1 = ov.verify(t, d, tokens, u, 0.0, "f32")
    r2 = ov.verify(t, d, tokens, u, 0.0, "f32", lenience=0.2)
    np.testing.assert_array_equal(r1.n_accepted, r2.n_accepted)
    np.testing.assert_array_equal(r1.next_token, r2.next_token)


# --------------------------------------------------- per-sequence draft counts

def test_ragged_tokens_per_round_follow_equation_1():
    rng = np.random.default_rng(34)
    V, gamma, rounds = 8, 7, 8000
    x = rng.standard_normal(V)
    p = np.exp(x) / np.exp(x).sum()
    y = rng.standard_normal(V)
    q = 0.7 * p + 0.3 * np.exp(y) / np.exp(y).sum()
    alpha = float(np.minimum(p, q).sum())
    for gb in (0, 1, 3, 7):
        gseq = np.full(rounds, gb)
        tokens = rng.choice(V, size=(rounds, gamma), p=q)
        u = np.clip(rng.random((rounds, gamma + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
        res = _run(np.broadcast_to(p, (rounds, gamma + 1, V)), np.broadcast_to(q, (rounds, gamma, V)),
                   tokens, u, gamma_seq=gseq)
        n_tok = res.n_accepted + 1
        assert n_tok.max() <= gb + 1
        want = float(exact.expected_tokens(F(alpha), gb))
        se = max(n_tok.std(), 1e-12) / np.sqrt(rounds)
        assert abs(n_tok.mean() - want) < 4 * se + 1e-12, (gb, n_tok.mean(), want)
        if gb:
            pmf = np.array([float(v) for v in exact.tokens_per_round_pmf(F(alpha), gb)])
            counts = np.bincount(n_tok, minlength=gb + 2)[1:]
            assert scipy.stats.chisquare(counts, rounds * pmf).pvalue > 1e-4


def test_ragged_gamma_zero_samples_the_first_target_row():
    rng = np.random.default_rng(35)
    V, gamma, trials = 5, 3, 200000
    p0 = np.array([0.1, 0.0, 0.45, 0.25, 0.2])
    rows = np.stack([p0] + [np.full(V, 0.2)] * gamma)            # p_0, then other rows
    q = np.full((gamma, V), 0.2)
    tokens = rng.integers(0, V, size=(trials, gamma))
    u = np.clip(rng.random((trials, gamma + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    res = _run(np.broadcast_to(rows, (trials, gamma + 1, V)), np.broadcast_to(q, (trials, gamma, V)),
               tokens, u, gamma_seq=np.zeros(trials, np.int64))
    assert np.all(res.n_accepted == 0)
    counts = np.bincount(res.next_token, minlength=V)
    assert counts[1] == 0
    sup = p0 > 0
    assert scipy.stats.chisquare(counts[sup], trials * p0[sup]).pvalue > 1e-4
    assert np.isnan(res.alpha).all()


def test_ragged_bonus_token_follows_row_gamma_b():
    """p_i = q_i for i < gamma_b keeps every draft, so the round's own token comes
    from the bonus row, which for a ragged sequence is target row gamma_b."""
    rng = np.random.default_rng(37)
    V, gamma, trials, gb = 5, 4, 200000, 2
    base = np.array([0.2, 0.2, 0.2, 0.2, 0.2])
    pb = np.array([0.05, 0.5, 0.0, 0.15, 0.3])
    tail = np.array([0.6, 0.1, 0.1, 0.1, 0.1])
    rows = np.stack([base, base, pb, tail, tail])
    q = np.tile(base, (gamma, 1))
    tokens = rng.integers(0, V, size=(trials, gamma))
    u = np.clip(rng.random((trials, gamma + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    res = _run(np.broadcast_to(rows, (trials, gamma + 1, V)), np.broadcast_to(q, (trials, gamma, V)),
               tokens, u, gamma_seq=np.full(trials, gb))
    assert np.all(res.n_accepted == gb)
    counts = np.bincount(res.next_token, minlength=V)
    assert counts[2] == 0
    sup = pb > 0
    assert scipy.stats.chisquare(counts[sup], trials * pb[sup]).pvalue > 1e-4


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_ragged_equals_unpadded_and_ignores_padding(T):
    rng = np.random.default_rng(36)
    B, G, V = 12, 5, 300
    t = (rng.standard_normal((B, G + 1, V)) * 2).astype(np.float32)
    d = (t[:, :G] + rng.standard_normal((B, G, V))).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, G))
    u = np.clip(rng.random((B, G + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    gseq = rng.integers(0, G + 1, size=B)
    # padding holds values that would poison any computation that read them
    tp, dp, kp = t.copy(), d.copy(), tokens.copy()
    for b in range(B):
        tp[b, gseq[b] + 1:] = np.nan
        dp[b, gseq[b]:] = np.nan
        kp[b, gseq[b]:] = -7
    res = ov.verify(tp, dp, kp, u, T, "f32", gamma_seq=gseq)
    for b in range(B):
        g = int(gseq[b])
        one = ov.verify(t[b:b + 1, :g + 1], d[b:b + 1, :g], tokens[b:b + 1, :g], u[b:b + 1, :g + 1], T, "f32")
        assert res.n_accepted[b] == one.n_accepted[0] and res.next_token[b] == one.next_token[0]
        np.testing.assert_array_equal(res.alpha[b, :g], one.alpha[0])
        np.testing.assert_array_equal(res.p_draft[b, :g], one.p_draft[0])
        assert np.isnan(res.alpha[b, g:]).all() and np.isnan(res.q_draft[b, g:]).all()
    with pytest.raises(ValueError):
        ov.verify(t, d, tokens, u, T, "f32", gamma_seq=np.full(B, G + 1))


# ------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("mutant", ["residual_unscaled", "lenience_in_numerator", "ragged_bonus_row"])
def test_planted_mistakes_in_the_extensions_are_caught(mutant, monkeypatch):
    orig_res, orig_ratio, orig_block = ov.residual_weights, ov.ratio_test, ov._verify_block
    if mutant == "residual_unscaled":
        monkeypatch.setattr(ov, "residual_weights", lambda p, q, l=1.0: orig_res(p, q, 1.0))
        # W3 at l = 1/2 rejects with probability 1/10, so its residual is used
        check = lambda: test_lenient_exact_enumeration("W3", F(1, 2))  # noqa: E731
    elif mutant == "lenience_in_numerator":
        monkeypatch.setattr(ov, "ratio_test", lambda px, qx, u, l=1.0: orig_ratio(px * l * l, qx, u, l))
        check = lambda: test_lenient_exact_enumeration("W100", F(1, 2))  # noqa: E731
    else:
        # the bonus row of a ragged sequence taken from the padded position gamma
        def block(target, draft, tokens, u, T, dtype, keep, lenience=1.0, gseq=None, *rest):
            r = orig_block(target, draft, tokens, u, T, dtype, keep, lenience, gseq, *rest)
            if gseq is not None:
                full = orig_block(target, draft, tokens, u, T, dtype, keep, lenience, None, *rest)
                allk = r.n_accepted == np.asarray(gseq)
                r.next_token = np.where(allk, full.next_token, r.next_token)
            return r
        monkeypatch.setattr(ov, "_verify_block", block)
        check = lambda: test_ragged_bonus_token_follows_row_gamma_b()  # noqa: E731
    with pytest.raises(AssertionError):
        check()
