"""Philox4x32-10 counter-based generator (host side, NumPy).

Written from the published definition in J. Salmon, M. Moraes, R. Dror and
D. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit
counter and a 2x32-bit key go through ten rounds.  Each round multiplies words 0
and 2 by two fixed odd constants and takes the high and low 32-bit halves.  It
then mixes the high halves with words 1 and 3 and the key by xor, and permutes
the words.  The key is advanced by two Weyl constants between rounds.

This module only produces random input for the verification step (the
uniforms the accept test and the final sample consume).  It holds none of the
verification arithmetic.
"""

from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo(a: np.uint64, b: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    prod = a * b.astype(np.uint64)
    return (prod >> np.uint64(32)).astype(np.uint32), (prod & _MASK32).astype(np.uint32)


def philox4x32_10(counter: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Apply Philox4x32-10 to counters.

    counter: uint32 array [..., 4]; key: uint32 array broadcastable to [..., 2].
    Returns uint32 [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint32)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint32), c.shape[:-1] + (2,))
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd:
                k0 = (k0 + _W0).astype(np.uint32)
                k1 = (k1 + _W1).astype(np.uint32)
            hi0, lo0 = _mulhilo(_M0, c0)
            hi1, lo1 = _mulhilo(_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def open_unit_f32(word: np.ndarray) -> np.ndarray:
    """Map a 32-bit word to a float32 in the open interval (0, 1).

    The top 23 bits k give u = (2k + 1) * 2^-24, exactly representable in
    float32, never 0 and never 1.
    """
    k = (np.asarray(word, dtype=np.uint32) >> np.uint32(9)).astype(np.float64)
    return ((2.0 * k + 1.0) * 2.0 ** -24).astype(np.float32)


def uniforms(seed: int, batch: int, count: int, offsets=None, tag: int = 0) -> np.ndarray:
    """Uniforms u[b][i] in (0, 1), float32 [batch, count].

    Counter = (offsets[b] + i, b, tag, 0), key = (seed & 0xffffffff, seed >> 32).
    `offsets` (one 32-bit start per row) defaults to zero.
    """
    if offsets is None:
        offsets = np.zeros(batch, dtype=np.uint64)
    offsets = np.asarray(offsets, dtype=np.uint64)
    b = np.arange(batch, dtype=np.uint64)[:, None]
    i = np.arange(count, dtype=np.uint64)[None, :]
    ctr = np.zeros((batch, count, 4), dtype=np.uint32)
    ctr[..., 0] = ((offsets[:, None] + i) & _MASK32).astype(np.uint32)
    ctr[..., 1] = np.broadcast_to(b, (batch, count)).astype(np.uint32)
    ctr[..., 2] = np.uint32(tag)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    return open_unit_f32(philox4x32_10(ctr, key)[..., 0])
