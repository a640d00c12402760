"""Pins of the oracle's exact-rational module against the numbers the pages print.

Fixtures live in tests/golden/, each entry naming the page and section it is
taken from.
"""

import json
import os
from fractions import Fraction as F

import pytest

from oracle import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _fr(xs):
    return [F(x) for x in xs]


EX = _load("worked_examples.json")
TOK = _load("expected_tokens.json")


@pytest.mark.parametrize("name", ["W3", "W4", "W100"])
def test_worked_example_overlap_and_emitted(name):
    ex = EX[name]
    p, q = _fr(ex["p"]), _fr(ex["q"])
    assert exact.overlap(p, q) == F(ex["alpha"])
    assert exact.overlap(p, q) == 1 - exact.total_variation(p, q)
    assert exact.emitted_distribution(p, q) == _fr(ex["emitted"])
    if "accepted_mass" in ex:
        assert exact.accepted_mass(p, q) == _fr(ex["accepted_mass"])
    if "residual_mass" in ex:
        assert exact.residual_mass(p, q) == _fr(ex["residual_mass"])
    if "residual_distribution" in ex:
        assert exact.residual_distribution(p, q) == _fr(ex["residual_distribution"])


def test_w3_rejection_probability():
    ex = EX["W3"]
    p, q = _fr(ex["p"]), _fr(ex["q"])
    assert 1 - exact.overlap(p, q) == F(ex["rejection"])
    assert sum(exact.residual_mass(p, q)) == F(ex["rejection"])


def test_w4_token_accounting():
    ex = EX["W4"]
    p, q = _fr(ex["p"]), _fr(ex["q"])
    acc = exact.accepted_mass(p, q)
    res = exact.residual_distribution(p, q)
    rejection = 1 - exact.overlap(p, q)
    assert p[1] / q[1] == F(ex["ratio_token_1"])
    assert acc[0] == F(ex["token_0_accepted"])
    assert rejection * res[0] == F(ex["token_0_from_rejection"])
    r_max = max(a / b for a, b in zip(p, q))
    assert 1 / r_max == F(ex["inverse_r_max"])
    # plain rejection sampling never accepts more often than speculative sampling
    assert 1 / r_max <= exact.overlap(p, q)


def test_special_cases():
    sc = EX["special_cases"]
    p, q = _fr(sc["equal"]["p"]), _fr(sc["equal"]["q"])
    assert exact.overlap(p, q) == F(sc["equal"]["alpha"])
    assert exact.residual_distribution(p, q) is None
    assert exact.emitted_distribution(p, q) == p
    p, q = _fr(sc["disjoint"]["p"]), _fr(sc["disjoint"]["q"])
    assert exact.overlap(p, q) == F(sc["disjoint"]["alpha"])
    assert exact.emitted_distribution(p, q) == _fr(sc["disjoint"]["emitted"])


def test_emitted_equals_target_for_random_rationals():
    import random
    rnd = random.Random(3)
    for _ in range(200):
        V = rnd.randint(1, 7)
        pw = [rnd.randint(0, 9) for _ in range(V)]
        qw = [rnd.randint(0, 9) for _ in range(V)]
        if sum(pw) == 0 or sum(qw) == 0:
            continue
        p = [F(x, sum(pw)) for x in pw]
        q = [F(x, sum(qw)) for x in qw]
        assert exact.emitted_distribution(p, q) == p
        assert exact.overlap(p, q) == 1 - exact.total_variation(p, q)


@pytest.mark.parametrize("case", TOK["eq1"]["cases"] + TOK["table1_speed"]["cases"])
def test_expected_tokens_printed_values(case):
    value = exact.expected_tokens(F(case["alpha"]), case["gamma"])
    printed = case.get("expected_tokens", case.get("speed"))
    assert round(float(value), case["decimals"]) == float(printed)


def test_expected_tokens_histogram_printed_values():
    h = TOK["eq1"]["histogram"]
    pmf = exact.tokens_per_round_pmf(F(h["alpha"]), h["gamma"])
    assert sum(pmf) == 1
    assert round(100 * float(pmf[-1])) == h["p_all_8_tokens_percent"]
    assert round(100 * float(pmf[0])) == h["p_one_token_percent"]
    mean = sum((k + 1) * pk for k, pk in enumerate(pmf))
    assert mean == exact.expected_tokens(F(h["alpha"]), h["gamma"])


def test_expected_tokens_saturation():
    for s in TOK["eq1"]["saturation"] + [TOK["ceiling"]]:
        a = F(s["alpha"])
        assert 1 / (1 - a) == F(s["limit"])
        # the finite-gamma value rises toward the ceiling and never reaches it
        vals = [exact.expected_tokens(a, g) for g in (1, 4, 16, 128)]
        assert all(x < y for x, y in zip(vals, vals[1:]))
        assert vals[-1] < F(s["limit"]) and F(s["limit"]) - vals[-1] < F(1, 100)


def test_positional_reduces_to_eq1():
    for a in (F(1, 3), F(3, 4), F(9, 10)):
        for g in (0, 1, 5, 9):
            assert exact.expected_tokens_positional([a] * g) == exact.expected_tokens(a, g)
    assert exact.expected_tokens(F(1), 4) == 5
