"""The seeded input generators: determinism, shapes, bf16 rounding and the
overlap levels the benchmark configurations are meant to have."""

import numpy as np

import workloads as W
from oracle import verify as ov


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.140625, 1e-40], np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert back.tolist()[:5] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 3.140625]
    y = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 5
    err = np.abs(W.bf16_bits_to_f32(W.f32_to_bf16_bits(y)) - y) / np.abs(y)
    assert err.max() <= 2 ** -8


def test_generators_deterministic_and_shaped():
    a = W.config1(3)
    b = W.config1(3)
    assert np.array_equal(a.target, b.target) and np.array_equal(a.tokens, b.tokens)
    assert a.target.shape == (1, 4, 32128) and a.draft.shape == (1, 3, 32128)
    assert a.tokens.dtype == np.int32 and a.uniforms.shape == (1, 4)
    c = W.config1(4)
    assert not np.array_equal(a.target, c.target)
    s = W.config3(0, B=3, V=4096)
    assert s.target.dtype == np.uint16 and s.target.shape == (3, 5, 4096)
    assert np.all((s.tokens >= 0) & (s.tokens < 4096))
    assert np.all((s.uniforms > 0) & (s.uniforms < 1))


def test_gumbel_tokens_follow_the_draft():
    # Gumbel-max draws x ~ softmax(l / T): check the frequency of a known row
    rng = np.random.default_rng(1)
    logits = np.log(np.array([0.1, 0.6, 0.3]))
    rows = np.broadcast_to(logits, (20000, 1, 3)).astype(np.float32)
    x = W.synth.gumbel_max_tokens(rows, 1.0, rng)[:, 0]
    freq = np.bincount(x, minlength=3) / len(x)
    assert np.abs(freq - [0.1, 0.6, 0.3]).max() < 0.015
    x0 = W.synth.gumbel_max_tokens(rows, 0.0, rng)[:, 0]
    assert np.all(x0 == 1)


def test_overlap_levels_of_configs():
    c1 = W.config1(0)
    r1 = ov.verify_case(c1)
    assert 0.5 < r1.alpha.mean() < 0.75
    c2 = W.config2(0, 1.0, rounds=4)
    r2 = ov.verify_case(c2)
    assert 0.55 < r2.alpha.mean() < 0.85
    c3 = W.config3(0, B=6, V=8192)
    r3 = ov.verify_case(c3)
    assert 0.2 < r3.alpha.min() and r3.alpha.max() < 0.99
    c5 = W.config5(0, B=6, V=16384)
    r5 = ov.verify_case(c5)
    assert 0.3 < r5.alpha.mean() < 0.8


def test_config5_confidently_wrong_rows():
    c = W.config5(1, B=40, V=2048, wrong_fraction=0.25)
    r = ov.verify_case(c)
    # a confidently-wrong row has overlap near 0 and its drafted token is rejected
    low = r.alpha < 0.02
    assert low.sum() >= 5
    dl = W.as_f32(c.draft, "bf16")
    tl = W.as_f32(c.target, "bf16")
    b, i = np.nonzero(low)
    # the drafted token is the target's minimum (bf16 rounding can create ties there)
    assert np.all(tl[b, i, c.tokens[b, i]] == tl[b, i].min(-1))
    assert np.all(dl[b, i].max(-1) >= tl[b, i].max(-1))


def test_config4_shapes_small():
    c = W.config4(0, B=2, gamma=3, d=64, V=512)
    assert c.hidden.shape == (8, 64) and c.w_target.shape == (64, 512)
    assert c.tokens.shape == (2, 3) and c.draft_hidden_rows().tolist() == [0, 1, 2, 4, 5, 6]
