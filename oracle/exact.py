"""Exact-rational statements of the method's single-step identities.

TEST INFRASTRUCTURE.  Page abbreviations are listed in oracle/__init__.py.

Everything here works on lists of fractions.Fraction and is exact:
  * the accepted mass min(p, q) and the residual max(0, p - q), and the fact
    that accepted mass plus rejection mass times the normalised residual gives
    back p ([LH] "Three candidates explain the acceptance rule"; [FI]
    "Speculative sampling: the accept/reject rule", Appendix A.1; [DB] "Show the
    short proof");
  * alpha = sum min(p, q) = 1 - TV(p, q) ([SD] "How often do we accept?");
  * expected tokens per round (1 - alpha^(gamma+1)) / (1 - alpha) and the
    distribution of tokens per round ([FI] "Tokens per target run, equation
    (1)"; [SD] "Expected yield per round");
  * the expectation for position-dependent acceptance, 1 + sum_k prod_{i<k} alpha_i,
    which follows from the same counting with a separate alpha per position.
"""

from __future__ import annotations

from fractions import Fraction as F


def accepted_mass(p, q):
    """Probability that a draft proposes x and it is kept: q(x) min(1, p/q) = min(p, q)."""
    return [min(a, b) for a, b in zip(p, q)]


def residual_mass(p, q):
    """Shortfall of the draft under the target: max(0, p - q), unnormalised."""
    return [max(a - b, F(0)) for a, b in zip(p, q)]


def overlap(p, q):
    return sum(accepted_mass(p, q), F(0))


def total_variation(p, q):
    return sum((abs(a - b) for a, b in zip(p, q)), F(0)) / 2


def residual_distribution(p, q):
    """max(0, p - q) / sum; None when the residual carries no mass (p == q)."""
    r = residual_mass(p, q)
    s = sum(r, F(0))
    return None if s == 0 else [x / s for x in r]


def emitted_distribution(p, q):
    """Distribution of the one token a single speculative step emits:
    kept proposals plus (rejection probability) x (normalised residual)."""
    acc = accepted_mass(p, q)
    rejection = 1 - sum(acc, F(0))
    if rejection == 0:
        return acc
    res = residual_distribution(p, q)
    return [a + rejection * r for a, r in zip(acc, res)]


def expected_tokens(alpha, gamma: int):
    """E[tokens per target run] with i.i.d. acceptance alpha: (1 - a^(g+1)) / (1 - a)."""
    alpha = F(alpha)
    if alpha == 1:
        return F(gamma + 1)
    return (1 - alpha ** (gamma + 1)) / (1 - alpha)


def tokens_per_round_pmf(alpha, gamma: int):
    """P(k tokens), k = 1..gamma+1: alpha^(k-1) (1 - alpha) for k <= gamma, alpha^gamma at gamma+1."""
    alpha = F(alpha)
    pmf = [alpha ** (k - 1) * (1 - alpha) for k in range(1, gamma + 1)]
    pmf.append(alpha ** gamma)
    return pmf


def expected_tokens_positional(alphas):
    """E[tokens] when draft i is kept with probability alphas[i], independently:
    1 + sum over k of the probability that the first k drafts are all kept."""
    total, run = F(1), F(1)
    for a in alphas:
        run *= F(a)
        total += run
    return total
