"""Pins of the top-k / top-p adjustment (oracle/adjust.py) and of the sampler run
on adjusted distributions.

  * top-k against torch's library top-k on the CPU (every value at least the k-th
    largest, ties included);
  * top-p against a brute-force statement of the definition over tiny rows, in
    fp64: the largest probability threshold pi whose set {p >= pi} holds at
    least top_p (a row whose decision lies within 1e-9 of a boundary, where the
    two fp64 summation orders may disagree, is exempt from the equality, not
    from the mass checks);
  * top-p after top-k renormalises over the top-k survivors;
  * the sampler then emits the adjusted target distribution ([FI] "The loop":
    the method treats the adjusted p and q as its distributions), checked by
    chi-squared;
  * top-k = 1 at T > 0 reduces to argmax mode for drafts that are the draft's
    argmax;
  * planted mistakes in the adjustment fail these pins.
"""

import numpy as np
import pytest
import scipy.stats
import torch

from oracle import adjust
from oracle import verify as ov


def _rows(rng, n, V, levels=None):
    x = rng.standard_normal((n, V)) * 2.0
    if levels:                      # quantise to force ties, as bf16 logits have
        x = np.round(x * levels) / levels
    return x


@pytest.mark.parametrize("V,k", [(10, 3), (50, 1), (50, 49), (300, 17), (300, 300), (300, 0)])
def test_topk_matches_library_topk(V, k):
    rng = np.random.default_rng(V * 7 + k)
    rows = _rows(rng, 20, V, levels=4)
    for r in rows:
        tau = adjust.topk_threshold(r, k)
        if k <= 0 or k >= V:
            assert tau == -np.inf
            continue
        kth = torch.topk(torch.from_numpy(r), k).values[-1].item()
        np.testing.assert_array_equal(r >= tau, r >= kth)
        assert (r >= tau).sum() >= k


def brute_topp(row, T, top_p, keep):
    """Largest pi with mass{p >= pi} >= top_p over the kept tokens, as a logit threshold."""
    z = np.where(keep, row, -np.inf)
    p = np.exp((z - z[keep].max()) / T)
    p /= p.sum()
    best = -np.inf
    for x in np.nonzero(keep)[0]:              # every candidate threshold is some token's probability
        if p[p >= p[x]].sum() >= top_p and p[x] > best:
            best = p[x]
    return z[keep & (p >= best)].min()


@pytest.mark.parametrize("top_p", [0.05, 0.3, 0.5, 0.9, 0.999])
@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_topp_matches_brute_force_definition(top_p, T):
    rng = np.random.default_rng(int(top_p * 1000) + int(T * 10))
    for r in _rows(rng, 30, 40, levels=3):
        tau, margin = adjust.topp_threshold(r, T, top_p)
        want = brute_topp(r, T, top_p, np.ones_like(r, bool))
        if margin > 1e-9:                        # not within fp64 summation-order rounding of a boundary
            assert tau == want
        kept = r >= tau
        p = np.exp((r - r.max()) / T)
        p /= p.sum()
        assert p[kept].sum() >= top_p - 1e-6
        # minimal: dropping the smallest kept tie group falls below top_p
        lowest = r[kept].min()
        assert p[kept & (r > lowest)].sum() < top_p + 1e-6


@pytest.mark.parametrize("k,top_p", [(5, 0.6), (12, 0.3), (3, 0.95)])
def test_topp_after_topk_renormalises_over_the_survivors(k, top_p):
    rng = np.random.default_rng(k)
    for r in _rows(rng, 30, 40, levels=5):
        tk = adjust.topk_threshold(r, k)
        tp, _ = adjust.topp_threshold(r, 1.0, top_p, tk)
        want = brute_topp(r, 1.0, top_p, r >= tk)
        assert max(tk, tp) == max(tk, want)


def test_disabled_filters_are_the_identity():
    rng = np.random.default_rng(3)
    B, G, V = 8, 3, 64
    t = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    d = (t[:, :G] + rng.standard_normal((B, G, V))).astype(np.float32)
    tok = rng.integers(0, V, size=(B, G))
    u = np.clip(rng.random((B, G + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    a = ov.verify(t, d, tok, u, 1.0, "f32")
    for k, p in ((0, 1.0), (V, 1.0), (-1, 1.5)):
        b = ov.verify(t, d, tok, u, 1.0, "f32", top_k=k, top_p=p)
        np.testing.assert_array_equal(a.n_accepted, b.n_accepted)
        np.testing.assert_array_equal(a.next_token, b.next_token)
        np.testing.assert_array_equal(a.alpha, b.alpha)


@pytest.mark.parametrize("k,top_p", [(3, 1.0), (0, 0.7), (4, 0.8)])
def test_sampler_emits_the_adjusted_target(k, top_p):
    rng = np.random.default_rng(11 + k)
    V, trials, T = 7, 100000, 1.0
    p_logit = rng.standard_normal(V) * 1.5
    q_logit = p_logit + rng.standard_normal(V)
    # adjusted distributions, written out directly from the definitions
    def adjusted(z):
        tk = adjust.topk_threshold(z, k)
        tp, _ = adjust.topp_threshold(z, T, top_p, tk)
        zz = np.where(z >= max(tk, tp), z, -np.inf)
        e = np.exp(zz - zz.max())
        return e / e.sum()
    pa, qa = adjusted(p_logit), adjusted(q_logit)
    tokens = rng.choice(V, size=(trials, 1), p=qa)
    u = np.clip(rng.random((trials, 2)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    res = ov.verify(np.broadcast_to(p_logit, (trials, 2, V)).astype(np.float32),
                    np.broadcast_to(q_logit, (trials, 1, V)).astype(np.float32), tokens, u, T, "f32",
                    top_k=k, top_p=top_p)
    emitted = np.where(res.n_accepted >= 1, tokens[:, 0], res.next_token)
    counts = np.bincount(emitted, minlength=V)
    assert np.all(counts[pa == 0] == 0)
    sup = pa > 0
    assert scipy.stats.chisquare(counts[sup], trials * pa[sup]).pvalue > 1e-4


def test_top1_reduces_to_argmax_mode():
    rng = np.random.default_rng(21)
    B, G, V = 40, 4, 100
    t = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    d = (t[:, :G] + rng.standard_normal((B, G, V))).astype(np.float32)
    tok = np.argmax(d, axis=-1)
    u = np.clip(rng.random((B, G + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    a = ov.verify(t, d, tok, u, 0.0, "f32")
    b = ov.verify(t, d, tok, u, 1.0, "f32", top_k=1)
    np.testing.assert_array_equal(a.n_accepted, b.n_accepted)
    np.testing.assert_array_equal(a.next_token, b.next_token)
    np.testing.assert_allclose(a.alpha, b.alpha, atol=0)


@pytest.mark.parametrize("mutant", ["topk_strict", "topp_exclusive", "topp_before_topk"])
def test_planted_mistakes_in_the_adjustment_are_caught(mutant, monkeypatch):
    orig_k, orig_p = adjust.topk_threshold, adjust.topp_threshold
    if mutant == "topk_strict":
        # keeps only values strictly above the k-th largest
        monkeypatch.setattr(adjust, "topk_threshold",
                            lambda row, k: np.nextafter(orig_k(row, k), np.inf) if 0 < k < row.shape[-1] else -np.inf)
        check = lambda: test_topk_matches_library_topk(300, 17)  # noqa: E731
    elif mutant == "topp_exclusive":
        # stops one tie group early (mass just below top_p)
        def early(row, T, top_p, tau_k=-np.inf):
            tau, mg = orig_p(row, T, top_p, tau_k)
            higher = row[(row > tau) & (row >= tau_k)]
            return (float(higher.min()) if higher.size else tau), mg
        monkeypatch.setattr(adjust, "topp_threshold", early)
        check = lambda: test_topp_matches_brute_force_definition(0.5, 1.0)  # noqa: E731
    else:
        # nucleus taken on the full distribution instead of the top-k survivors
        monkeypatch.setattr(adjust, "topp_threshold", lambda row, T, top_p, tau_k=-np.inf: orig_p(row, T, top_p))
        check = lambda: test_topp_after_topk_renormalises_over_the_survivors(5, 0.6)  # noqa: E731
    with pytest.raises(AssertionError):
        check()
