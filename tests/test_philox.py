"""Philox4x32-10 input generator: known-answer vectors and the uniform mapping."""

import numpy as np

from workloads.philox import open_unit_f32, philox4x32_10, uniforms

# Known-answer vectors distributed with the Random123 reference implementation of
# Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
KAT = [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


def test_known_answer_vectors():
    for ctr, key, want in KAT:
        got = philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
        assert [int(x) for x in got] == want


def test_batched_matches_single():
    rng = np.random.default_rng(1)
    ctr = rng.integers(0, 2 ** 32, size=(17, 4), dtype=np.uint64).astype(np.uint32)
    key = np.array([12345, 678], np.uint32)
    batched = philox4x32_10(ctr, key)
    for r in range(ctr.shape[0]):
        assert np.array_equal(batched[r], philox4x32_10(ctr[r], key))


def test_open_unit_interval_and_exactness():
    words = np.array([0, 1, 511, 512, 0xFFFFFFFF, 0x80000000], np.uint32)
    u = open_unit_f32(words)
    assert np.all(u > 0) and np.all(u < 1)
    assert u[0] == np.float32(2.0 ** -24)
    assert u[4] == np.float32(1 - 2.0 ** -24)
    # (2k+1) 2^-24 with k < 2^23 is exact in float32
    k = (words >> 9).astype(np.float64)
    assert np.array_equal(u.astype(np.float64), (2 * k + 1) * 2.0 ** -24)


def test_uniforms_shape_offsets_and_moments():
    u = uniforms(7, 1000, 9)
    assert u.shape == (1000, 9) and u.dtype == np.float32
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005
    # an offset of +1 shifts the counter stream by one position
    u0 = uniforms(7, 3, 5, offsets=np.array([0, 10, 20]))
    u1 = uniforms(7, 3, 5, offsets=np.array([1, 11, 21]))
    assert np.array_equal(u0[:, 1:], u1[:, :-1])
