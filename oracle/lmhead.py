"""fp64 LM-head product for the fused LM-head + verify workload.

TEST INFRASTRUCTURE.  Page abbreviations are listed in oracle/__init__.py.

The target pass ends in a matrix product of the hidden state at each of the
gamma+1 positions with the output embedding; during decoding every weight is
read once and used once, which is why the product is memory-bound ([FI]
"Decoding waits on memory, not arithmetic").  Here the product is written
directly: logits[m, v] = sum_k hidden[m, k] * W[k, v], with the bf16 inputs
widened exactly to float64.
"""

from __future__ import annotations

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def logits(hidden_bits: np.ndarray, w_bits: np.ndarray, cols: slice | None = None,
           col_block: int = 8192) -> np.ndarray:
    """hidden [M, d] (bf16 bits) @ W [d, V] (bf16 bits) in float64 -> [M, V] (or the given columns)."""
    h = widen_bf16(hidden_bits)
    V = w_bits.shape[1]
    lo, hi = (0, V) if cols is None else (cols.start or 0, cols.stop if cols.stop is not None else V)
    out = np.empty((h.shape[0], hi - lo))
    for c in range(lo, hi, col_block):
        e = min(hi, c + col_block)
        out[:, c - lo:e - lo] = h @ widen_bf16(w_bits[:, c:e])
    return out


def abs_error_bound(hidden_bits: np.ndarray, w_bits: np.ndarray, cols: slice | None = None,
                    unit_roundoff: float = 2.0 ** -24) -> np.ndarray:
    """Worst-case rounding bound of an fp32-accumulated product: d * u * sum_k |h_k w_kv|.

    Products of two bf16 values are exact in fp32, so only the d additions round.
    """
    h = np.abs(widen_bf16(hidden_bits))
    V = w_bits.shape[1]
    lo, hi = (0, V) if cols is None else (cols.start or 0, cols.stop if cols.stop is not None else V)
    d = h.shape[1]
    return d * unit_roundoff * (h @ np.abs(widen_bf16(w_bits[:, lo:hi])))
