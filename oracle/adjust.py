"""Top-k and top-p (nucleus) adjustment of logit rows, fp64.

TEST INFRASTRUCTURE, like the rest of oracle/.

[FI] "The loop: draft, verify in one pass, keep a prefix": p and q are the
models' next-token distributions already adjusted for the sampling method in
use; top-k and nucleus sampling zero the tail and renormalise, and the method
then treats the adjusted p and q as its distributions.  [NZ] "5. Sampling and
evaluation": temperature, top-k and top-p must be applied consistently with the
acceptance rule, so the same settings adjust the target and the draft rows.

Readings taken where the pages are silent (each is listed in the design notes):
  * Order: temperature, then top-k, then top-p on the distribution renormalised
    over the top-k survivors.
  * Ties are kept: top-k keeps every token whose logit is at least the k-th
    largest logit; top-p keeps every token whose probability is at least that
    of the last token the descending walk needs, so the kept set is a set of
    whole tie groups and never depends on an order among equal values.
  * top-p keeps the smallest such set whose mass reaches top_p (at least the
    most likely tie group).  top_k <= 0 or top_k >= V, and top_p >= 1, disable
    the filter.
  * A filter is a per-row logit threshold tau: a token is kept when its logit
    is >= tau (the logit order is the probability order at any T > 0), and
    dropped tokens get logit -inf, i.e. probability 0.
  * In argmax mode (T = 0) the filters change nothing: the argmax group is
    always kept.
"""

from __future__ import annotations

import numpy as np


def topk_threshold(row: np.ndarray, k: int) -> float:
    """The k-th largest value of a row (ties kept), or -inf when k disables the filter."""
    V = row.shape[-1]
    if k <= 0 or k >= V:
        return -np.inf
    return float(np.partition(row, V - k)[V - k])


def topp_threshold(row: np.ndarray, temperature: float, top_p: float, tau_k: float = -np.inf):
    """Logit threshold of the nucleus of softmax(row / T) restricted to row >= tau_k.

    The tie groups (equal logits) are walked from the most likely down, and
    the walk stops at the first group where the cumulative mass, normalised
    over the kept tokens, reaches top_p; that group's logit is the threshold.

    Returns (tau_p, margin): tau_p is the smallest logit kept; margin is the
    distance of top_p from the two cumulative masses the decision compares it
    with (the sum before and after the boundary tie group), as a fraction of
    the total.  A decision taken in other arithmetic can only differ when its
    error in those normalised sums reaches the margin."""
    if top_p >= 1.0 or temperature <= 0.0:
        return -np.inf, np.inf
    kept = row[(row >= tau_k) & (row != -np.inf)]
    vals, counts = np.unique(kept, return_counts=True)          # ascending distinct logits
    vals, counts = vals[::-1], counts[::-1]                      # descending
    m = vals[0]
    w = counts * np.exp((vals - m) / temperature)                # mass of each tie group
    cum = np.cumsum(w) / w.sum()
    hit = cum >= top_p
    j = int(np.argmax(hit)) if hit.any() else len(cum) - 1
    before = cum[j - 1] if j > 0 else 0.0
    margin = min(abs(cum[j] - top_p), abs(top_p - before))
    return float(vals[j]), float(margin)


def thresholds(rows: np.ndarray, temperature: float, top_k: int, top_p: float):
    """Per-row keep thresholds for rows [..., V] (fp64 logits) and the top-p margins."""
    flat = rows.reshape(-1, rows.shape[-1])
    tau = np.full(flat.shape[0], -np.inf)
    margin = np.full(flat.shape[0], np.inf)
    for r in range(flat.shape[0]):
        tk = topk_threshold(flat[r], top_k)
        tp, mg = topp_threshold(flat[r], temperature, top_p, tk)
        tau[r] = max(tk, tp)
        margin[r] = mg
    return tau.reshape(rows.shape[:-1]), margin.reshape(rows.shape[:-1])


def apply(rows: np.ndarray, tau: np.ndarray) -> np.ndarray:
    """Rows with every logit below its row's threshold replaced by -inf."""
    return np.where(rows >= tau[..., None], rows, -np.inf)
