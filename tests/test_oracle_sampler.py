"""The oracle as a whole sampler: the emitted token must be distributed as the
target p ([SD] "Exactness"; [FI] "Speculative sampling: the accept/reject rule").

Four kinds of pin:
  * exact enumeration: for gamma = 1 and the pages' worked examples, every drafted
    token x is weighted by q(x) and the two uniforms run over a midpoint grid that
    never touches a decision boundary, so the emitted frequencies equal p to
    rounding;
  * chi-squared over 10^6 seeded trials;
  * Monte Carlo of the accepted-prefix length against equation (1) and its
    per-round distribution ([FI] "Tokens per target run, equation (1)");
  * planted mistakes: each plausible error in an oracle step makes one of the
    pins above fail.
"""

import json
import os
from fractions import Fraction as F

import numpy as np
import pytest
import scipy.stats

from oracle import exact
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
    EX = json.load(f)


def _probs(xs):
    return np.array([float(F(x)) for x in xs])


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def _run(p_rows, q_rows, tokens, u, T=1.0):
    """Oracle on probability rows given as float64 logits log(p) (batch of identical rows)."""
    target = _log(p_rows).astype(np.float32)
    draft = _log(q_rows).astype(np.float32)
    return ov.verify(target, draft, tokens, u, T, "f32")


def _first_emitted(res, tokens):
    """First token a round emits: x_0 if kept, else the target's own token."""
    return np.where(res.n_accepted >= 1, tokens[:, 0], res.next_token)


def grid_emitted_distribution(p, q, N=600):
    """Exact enumeration for gamma = 1: sum_x q(x) * frequency over an N x N midpoint grid."""
    V = len(p)
    g = (np.arange(N) + 0.5) / N
    u0, u1 = np.meshgrid(g, g, indexing="ij")
    u = np.stack([u0.ravel(), u1.ravel()], axis=-1).astype(np.float32)
    M = u.shape[0]
    out = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        tokens = np.full((M, 1), x, np.int64)
        p_rows = np.broadcast_to(p, (M, 2, V))
        q_rows = np.broadcast_to(q, (M, 1, V))
        res = _run(p_rows, q_rows, tokens, u)
        emitted = _first_emitted(res, tokens)
        out += q[x] * np.bincount(emitted, minlength=V) / M
    return out


def _grid_ok(name, N=600):
    p, q = _probs(EX[name]["p"]), _probs(EX[name]["q"])
    return np.abs(grid_emitted_distribution(p, q, N) - p).max() < 1e-6


@pytest.mark.parametrize("name", ["W3", "W4", "W100"])
def test_exact_enumeration_emits_target(name):
    # 600 is a multiple of every denominator in the three examples' ratios and
    # residual CDFs, so the midpoint grid gives the exact probabilities.
    p, q = _probs(EX[name]["p"]), _probs(EX[name]["q"])
    dist = grid_emitted_distribution(p, q)
    np.testing.assert_allclose(dist, p, atol=1e-12)
    assert np.all(dist[p == 0] == 0)


def _chi2_first_token(p, q, trials, seed):
    rng = np.random.default_rng(seed)
    V = len(p)
    tokens = rng.choice(V, size=(trials, 1), p=q)
    u = rng.random((trials, 2)).astype(np.float32)
    u = np.clip(u, np.float32(2 ** -24), np.float32(1 - 2 ** -24))
    res = _run(np.broadcast_to(p, (trials, 2, V)), np.broadcast_to(q, (trials, 1, V)), tokens, u)
    counts = np.bincount(_first_emitted(res, tokens), minlength=V)
    support = p > 0
    stat, pval = scipy.stats.chisquare(counts[support], trials * p[support])
    return counts, pval


@pytest.mark.parametrize("name", ["W3", "W4", "W100"])
def test_chi_squared_million_trials(name):
    p, q = _probs(EX[name]["p"]), _probs(EX[name]["q"])
    counts, pval = _chi2_first_token(p, q, 10 ** 6, seed=11)
    assert pval > 1e-4, (counts, pval)
    assert np.all(counts[p == 0] == 0)


def test_chi_squared_uniform_draft_and_disjoint_support():
    # a uniform draft still yields an exact sampler ([SD] "Exactness", assumptions)
    p = np.array([0.05, 0.6, 0.0, 0.25, 0.1])
    q = np.full(5, 0.2)
    counts, pval = _chi2_first_token(p, q, 200000, seed=12)
    assert pval > 1e-4 and counts[2] == 0
    # disjoint supports: every draft is rejected and the output is still p
    p = np.array([0.7, 0.3, 0.0, 0.0])
    q = np.array([0.0, 0.0, 0.5, 0.5])
    trials = 100000
    rng = np.random.default_rng(13)
    tokens = rng.choice(4, size=(trials, 1), p=q)
    u = rng.random((trials, 2)).astype(np.float32)
    res = _run(np.broadcast_to(p, (trials, 2, 4)), np.broadcast_to(q, (trials, 1, 4)), tokens, u)
    assert np.all(res.n_accepted == 0)
    counts = np.bincount(res.next_token, minlength=4)
    assert counts[2] == counts[3] == 0
    assert scipy.stats.chisquare(counts[:2], trials * p[:2]).pvalue > 1e-4


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((300, 6, 50)).astype(np.float32)
    tokens = rng.integers(0, 50, size=(300, 5))
    u = rng.random((300, 6)).astype(np.float32)
    res = ov.verify(x, x[:, :5].copy(), tokens, u, 0.8, "f32")
    assert np.all(res.n_accepted == 5)
    np.testing.assert_allclose(res.alpha, 1.0, atol=1e-12)


def _positional_rounds(p_rows, q_rows, rounds, seed):
    """Rounds with fixed per-position (p_i, q_i); drafts x_i ~ q_i independently."""
    rng = np.random.default_rng(seed)
    gamma, V = q_rows.shape
    tokens = np.stack([rng.choice(V, size=rounds, p=q_rows[i]) for i in range(gamma)], axis=1)
    u = np.clip(rng.random((rounds, gamma + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    res = _run(np.broadcast_to(p_rows, (rounds,) + p_rows.shape),
               np.broadcast_to(q_rows, (rounds,) + q_rows.shape), tokens, u)
    return tokens, res


def _random_dists(rng, k, V, sharp=1.0):
    x = rng.standard_normal((k, V)) * sharp
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_accept_length_matches_equation_1():
    # identical (p, q) at every position -> i.i.d. acceptance with alpha = overlap
    rng = np.random.default_rng(15)
    V, gamma, rounds = 8, 7, 10 ** 4
    p = _random_dists(rng, 1, V)[0]
    q = 0.7 * p + 0.3 * _random_dists(rng, 1, V)[0]
    alpha = float(np.minimum(p, q).sum())
    tokens, res = _positional_rounds(np.tile(p, (gamma + 1, 1)), np.tile(q, (gamma, 1)), rounds, 16)
    n_tok = res.n_accepted + 1
    want = float(exact.expected_tokens(F(alpha), gamma))
    pmf = np.array([float(x) for x in exact.tokens_per_round_pmf(F(alpha), gamma)])
    se = n_tok.std() / np.sqrt(rounds)
    assert abs(n_tok.mean() - want) < 4 * se, (n_tok.mean(), want, se)
    counts = np.bincount(n_tok, minlength=gamma + 2)[1:]
    assert scipy.stats.chisquare(counts, rounds * pmf).pvalue > 1e-4
    np.testing.assert_allclose(res.alpha, alpha, atol=1e-12)


def test_accept_length_positional_alpha():
    # position-dependent overlaps: E[tokens] = 1 + sum_k prod_{i<k} alpha_i
    rng = np.random.default_rng(17)
    V, gamma, rounds = 6, 5, 40000
    p = _random_dists(rng, gamma + 1, V, 1.5)
    mix = np.linspace(0.95, 0.3, gamma)[:, None]
    q = mix * p[:gamma] + (1 - mix) * _random_dists(rng, gamma, V, 1.5)
    alphas = np.minimum(p[:gamma], q).sum(axis=-1)
    tokens, res = _positional_rounds(p, q, rounds, 18)
    n_tok = res.n_accepted + 1
    want = float(exact.expected_tokens_positional([F(a) for a in alphas]))
    se = n_tok.std() / np.sqrt(rounds)
    assert abs(n_tok.mean() - want) < 4 * se


def test_each_emitted_position_follows_its_target_row():
    # conditional on a round reaching position k, the token it emits there is ~ p_k
    rng = np.random.default_rng(19)
    V, gamma, rounds = 5, 3, 300000
    p = _random_dists(rng, gamma + 1, V, 1.2)
    q = 0.5 * p[:gamma] + 0.5 * _random_dists(rng, gamma, V, 1.2)
    tokens, res = _positional_rounds(p, q, rounds, 20)
    n = res.n_accepted
    for k in range(gamma + 1):
        reach = n >= k
        emitted = np.where(n[reach] > k, tokens[reach, min(k, gamma - 1)], res.next_token[reach])
        counts = np.bincount(emitted, minlength=V)
        assert scipy.stats.chisquare(counts, reach.sum() * p[k]).pvalue > 1e-4, k


def test_argmax_mode_is_greedy_prefix():
    # at T = 0 the step keeps the drafts that equal the target argmax and emits the
    # target's argmax at the first mismatch ([LH] "What does 'unchanged output' mean?")
    rng = np.random.default_rng(21)
    B, gamma, V = 400, 4, 7
    target = rng.integers(-2, 3, size=(B, gamma + 1, V)).astype(np.float32)
    draft = rng.integers(-2, 3, size=(B, gamma, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, gamma))
    greedy = target.argmax(-1)
    tokens = np.where(rng.random((B, gamma)) < 0.6, greedy[:, :gamma], tokens)
    res = ov.verify(target, draft, tokens, np.full((B, gamma + 1), 0.5, np.float32), 0.0, "f32")
    for b in range(B):
        k = 0
        while k < gamma and tokens[b, k] == greedy[b, k]:
            k += 1
        assert res.n_accepted[b] == k and res.next_token[b] == greedy[b, k]
        for i in range(gamma):
            assert res.alpha[b, i] == float(greedy[b, i] == draft[b, i].argmax())


def test_low_temperature_limit_matches_argmax_mode():
    # as T -> 0 the overlap tends to [argmaxes agree] and the sample to the target argmax
    rng = np.random.default_rng(22)
    B, gamma, V = 200, 3, 40
    # distinct logits 0.5 apart, so no near-tie survives a cold temperature
    target = (0.5 * rng.permuted(np.tile(np.arange(V), (B, gamma + 1, 1)), axis=-1)).astype(np.float32)
    draft = (0.5 * rng.permuted(np.tile(np.arange(V), (B, gamma, 1)), axis=-1)).astype(np.float32)
    draft = np.where(rng.random((B, gamma, 1)) < 0.5, target[:, :gamma], draft)
    tokens = draft.argmax(-1)
    u = rng.random((B, gamma + 1)).astype(np.float32)
    cold = ov.verify(target, draft, tokens, u, 1e-3, "f32")
    zero = ov.verify(target, draft, tokens, u, 0.0, "f32")
    assert np.array_equal(cold.n_accepted, zero.n_accepted)
    assert np.array_equal(cold.next_token, zero.next_token)
    np.testing.assert_allclose(cold.alpha, zero.alpha, atol=1e-9)


def test_degenerate_shapes():
    rng = np.random.default_rng(23)
    # gamma = 0: plain sampling from p_0
    p = np.array([0.2, 0.5, 0.3])
    u = np.array([[0.1], [0.25], [0.69], [0.71], [0.999]], np.float32)
    res = _run(np.broadcast_to(p, (5, 1, 3)), np.zeros((5, 0, 3)), np.zeros((5, 0), np.int64), u)
    assert res.n_accepted.tolist() == [0] * 5 and res.next_token.tolist() == [0, 1, 1, 2, 2]
    # V = 1: the only token is always emitted
    res = ov.verify(np.zeros((4, 3, 1), np.float32), np.zeros((4, 2, 1), np.float32),
                    np.zeros((4, 2), np.int64), rng.random((4, 3)).astype(np.float32), 1.0, "f32")
    assert res.n_accepted.tolist() == [2] * 4 and res.next_token.tolist() == [0] * 4
    # B = 0
    res = ov.verify(np.zeros((0, 3, 5), np.float32), np.zeros((0, 2, 5), np.float32),
                    np.zeros((0, 2), np.int64), np.zeros((0, 3), np.float32), 1.0, "f32")
    assert res.n_accepted.shape == (0,)


def test_confidently_wrong_draft_rejected():
    # the draft puts almost all mass on a token the target almost never picks
    V = 16
    tl = np.zeros((1, 2, V), np.float32)
    tl[0, :, 3] = -40.0
    dl = np.zeros((1, 1, V), np.float32)
    dl[0, 0, 3] = 30.0
    res = ov.verify(tl, dl, np.array([[3]]), np.array([[1e-6, 0.5]], np.float32), 1.0, "f32")
    assert res.n_accepted[0] == 0 and res.next_token[0] != 3
    assert res.alpha[0, 0] < 1e-10


# ------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("mutant", ["residual_sign", "ratio_inverted", "prefix_off_by_one",
                                    "overlap_max", "cdf_ge_first", "softmax_no_temperature",
                                    "argmax_last"])
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    orig = {k: getattr(ov, k) for k in ("residual_weights", "ratio_test", "accepted_prefix",
                                         "overlap", "inverse_cdf", "softmax", "argmax_first")}
    if mutant == "residual_sign":
        monkeypatch.setattr(ov, "residual_weights", lambda p, q, l=1.0: np.maximum(0.0, l * q - p))
    elif mutant == "ratio_inverted":
        monkeypatch.setattr(ov, "ratio_test", lambda px, qx, u, l=1.0: orig["ratio_test"](qx, px, u, l))
    elif mutant == "prefix_off_by_one":
        monkeypatch.setattr(ov, "accepted_prefix",
                            lambda a: np.minimum(orig["accepted_prefix"](a) + 1, a.shape[-1]))
    elif mutant == "overlap_max":
        monkeypatch.setattr(ov, "overlap", lambda p, q: np.maximum(p, q).sum(-1))
    elif mutant == "cdf_ge_first":
        def ge(probs, u):
            cdf = np.cumsum(probs, axis=-1)
            return np.argmax(cdf >= u[:, None], axis=-1), cdf
        monkeypatch.setattr(ov, "inverse_cdf", ge)
    elif mutant == "softmax_no_temperature":
        monkeypatch.setattr(ov, "softmax", lambda rows, T: orig["softmax"](rows, 1.0))
    elif mutant == "argmax_last":
        monkeypatch.setattr(ov, "argmax_first",
                            lambda r: r.shape[-1] - 1 - np.argmax(r[..., ::-1], axis=-1))

    caught = []
    caught.append(not all(_grid_ok(n, N=300) for n in ("W3", "W4", "W100")))
    p4, q4 = _probs(EX["W4"]["p"]), _probs(EX["W4"]["q"])
    res = _run(p4[None, None].repeat(2, 1), q4[None, None], np.array([[1]]),
               np.array([[0.5, 0.5]], np.float32))
    caught.append(abs(res.alpha[0, 0] - 0.75) > 1e-9)
    # strict ">" on an exact CDF edge: w = [0.5, 0, 0.5], u = 0.5 must give token 2
    edge = ov.inverse_cdf(np.array([[0.5, 0.0, 0.5]]), np.array([0.5]))[0][0]
    caught.append(edge != 2)
    # temperature: p = softmax(l / 0.5) at a known logit gap
    tl = np.array([[[0.0, np.log(3.0)], [0.0, 0.0]]], np.float32)
    dl = np.array([[[0.0, 0.0]]], np.float32)
    res = ov.verify(tl, dl, np.array([[1]]), np.array([[0.5, 0.5]], np.float32), 0.5, "f32")
    caught.append(abs(res.p_draft[0, 0] - 0.9) > 1e-6)
    # argmax ties: lowest index
    res = ov.verify(np.zeros((1, 2, 4), np.float32), np.zeros((1, 1, 4), np.float32),
                    np.array([[0]]), np.full((1, 2), 0.5, np.float32), 0.0, "f32")
    caught.append(not (res.n_accepted[0] == 1 and res.next_token[0] == 0))
    assert any(caught), mutant
