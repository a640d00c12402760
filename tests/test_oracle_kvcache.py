"""Pins of the KV-cache crop (oracle/kvcache.py).

[FI] "The loop: draft, verify in one pass, keep a prefix", the KV-cache
paragraph: after the accept test the entries beyond the accepted prefix are
discarded.  [LH] "Fix the benchmark conditions first": the cache follows the
committed prefix, and rejected state (with paged storage, whole pages) goes
back to the pool.

The expected outputs of the small cases are written out by hand below.
Invariants on random cases: bytes outside the discarded ranges are untouched,
the discarded ranges are zero, no page is lost or duplicated between the block
tables and the free list, and a -1 sequence is untouched.  Planted mistakes
fail the pins.
"""

import numpy as np
import pytest

from oracle import kvcache as kv


def test_contiguous_hand_case():
    # B=2, H=1, S_max=8, D=1; committed lengths 3 and 5; the pass wrote 3
    # entries (positions 3,4,5 and 5,6,7); 1 and 3 drafts accepted
    cache = np.arange(1, 17, dtype=np.int32).reshape(2, 1, 8, 1)
    new = kv.crop_contiguous([cache], [3, 5], [1, 3], appended=3, keep_extra=0, clear=True)
    assert new.tolist() == [4, 8]
    assert cache[0, 0, :, 0].tolist() == [1, 2, 3, 4, 0, 0, 7, 8]      # positions 4, 5 discarded
    assert cache[1, 0, :, 0].tolist() == [9, 10, 11, 12, 13, 14, 15, 16]  # every write kept


def test_contiguous_keep_extra_and_no_clear():
    # the pass also wrote the previous step's final token (keep_extra = 1):
    # committed 2, wrote positions 2..5 (appended 4), 0 accepted -> length 3
    cache = np.ones((1, 2, 6, 2), np.float32)
    new = kv.crop_contiguous([cache], [2], [0], appended=4, keep_extra=1, clear=True)
    assert new.tolist() == [3]
    assert (cache[0, :, 3:6] == 0).all() and (cache[0, :, :3] == 1).all()
    cache2 = np.ones((1, 2, 6, 2), np.float32)
    new2 = kv.crop_contiguous([cache2], [2], [0], appended=4, keep_extra=1, clear=False)
    assert new2.tolist() == [3] and (cache2 == 1).all()


def test_contiguous_failed_sequence_and_capacity():
    cache = np.full((2, 1, 4, 1), 7, np.int16)
    # sequence 0 reported -1: untouched; sequence 1 wrote past S_max = 4
    new = kv.crop_contiguous([cache], [1, 2], [-1, 0], appended=3, keep_extra=0, clear=True)
    assert new.tolist() == [1, 2]
    assert (cache[0] == 7).all()
    assert cache[1, 0, :, 0].tolist() == [7, 7, 0, 0]


def test_paged_hand_case():
    # page_size 2, H = D = 1; pages 0..5 hold the value 10*page + slot
    P = 2
    cache = np.array([[10 * p, 10 * p + 1] for p in range(6)], np.int32).reshape(6, P, 1, 1)
    table = np.array([[0, 3, 5, -1], [1, 2, -1, -1]], np.int32)
    free = np.full(6, -9, np.int32)
    free[0] = 4                                   # one page already free
    new, count = kv.crop_paged([cache], table, [3, 1], [0, 2], appended=3, keep_extra=0, clear=True,
                               free_pages=free, free_count=1, page_size=P, num_pages=6)
    assert new.tolist() == [3, 3]
    # sequence 0 keeps 3 positions = blocks 0, 1; block 2 (page 5) is released
    assert table.tolist() == [[0, 3, -1, -1], [1, 2, -1, -1]]
    assert count == 2 and free.tolist() == [4, 5, -9, -9, -9, -9]
    # cleared: seq 0 positions 3, 4, 5 -> page 3 slot 1, page 5 slots 0 and 1;
    #          seq 1 position 3 -> page 2 slot 1
    want = np.array([[10 * p, 10 * p + 1] for p in range(6)], np.int32)
    want[3, 1] = want[5, 0] = want[5, 1] = want[2, 1] = 0
    assert cache.reshape(6, P).tolist() == want.tolist()


def test_paged_release_order_and_failed_sequence():
    # sequences in order, blocks ascending; a -1 sequence keeps its pages
    table = np.array([[0, 1, 2, 3], [4, 5, 6, 7], [-1, -1, -1, -1]], np.int32)
    free = np.full(8, -1, np.int32)
    new, count = kv.crop_paged([], table, [1, 4, 0], [0, -1, 2], appended=4, keep_extra=0, clear=False,
                               free_pages=free, free_count=0, page_size=4, num_pages=8)
    assert new.tolist() == [1, 4, 2]
    assert table.tolist() == [[0, -1, -1, -1], [4, 5, 6, 7], [-1, -1, -1, -1]]
    assert count == 3 and free[:3].tolist() == [1, 2, 3]


def _random_paged(rng, B=5, max_blocks=6, P=4, H=2, D=3):
    num_pages = B * max_blocks + 3
    ids = rng.permutation(num_pages)
    table = np.full((B, max_blocks), -1, np.int32)
    seq_len = rng.integers(0, (max_blocks - 2) * P, size=B)
    appended = 5
    k = 0
    for b in range(B):
        used = -(-(seq_len[b] + appended) // P)
        for j in range(min(used, max_blocks)):
            table[b, j] = ids[k]
            k += 1
    free = np.full(num_pages, -1, np.int32)
    free[:num_pages - k] = ids[k:]
    caches = [rng.integers(1, 100, size=(num_pages, P, H, D)).astype(np.int32) for _ in range(2)]
    return caches, table, seq_len, appended, free, num_pages - k


@pytest.mark.parametrize("seed", range(6))
def test_paged_invariants(seed):
    rng = np.random.default_rng(seed)
    caches, table, seq_len, appended, free, count = _random_paged(rng)
    before_pages = set(table[table >= 0].tolist()) | set(free[:count].tolist())
    orig = [c.copy() for c in caches]
    t0 = table.copy()
    n = rng.integers(-1, 5, size=len(seq_len))
    P = caches[0].shape[1]
    new, count2 = kv.crop_paged(caches, table, seq_len, n, appended, 0, True, free, count, P, caches[0].shape[0])
    after_pages = set(table[table >= 0].tolist()) | set(free[:count2].tolist())
    assert before_pages == after_pages                                     # nothing lost
    assert len(table[table >= 0]) + count2 == len(before_pages)           # nothing duplicated
    for b in range(len(seq_len)):
        if n[b] < 0:
            assert (table[b] == t0[b]).all() and new[b] == seq_len[b]
            continue
        assert new[b] == seq_len[b] + n[b]
        assert (table[b, -(-new[b] // P):] == -1).all()
        assert (table[b, :-(-new[b] // P)] == t0[b, :-(-new[b] // P)]).all()
    # every changed byte is a zeroed discarded entry
    for c, o in zip(caches, orig):
        changed = np.argwhere((c != o).any(axis=(2, 3)))
        for page, slot in changed:
            assert (c[page, slot] == 0).all()
            b, j = np.argwhere(t0 == page)[0]
            s = j * P + slot
            assert n[b] >= 0 and seq_len[b] + n[b] <= s < seq_len[b] + appended


@pytest.mark.parametrize("mutant", ["keep_one_more", "release_kept_block", "clear_kept"])
def test_planted_mistakes_in_the_crop_are_caught(mutant, monkeypatch):
    orig_c, orig_p = kv.crop_contiguous, kv.crop_paged
    if mutant == "keep_one_more":
        def bad(caches, seq_len, n, appended, keep_extra, clear):
            return orig_c(caches, seq_len, np.asarray(n) + 1, appended, keep_extra, clear)
        monkeypatch.setattr(kv, "crop_contiguous", bad)
        check = test_contiguous_hand_case
    elif mutant == "release_kept_block":
        def bad(caches, table, seq_len, n, appended, keep_extra, clear, free_pages, free_count, page_size,
                num_pages):
            new, cnt = orig_p(caches, table, seq_len, n, appended, keep_extra, clear, free_pages, free_count,
                              page_size, num_pages)
            for b in range(table.shape[0]):        # also release the last kept block
                j = -(-int(new[b]) // page_size) - 1
                if j >= 0 and table[b, j] >= 0:
                    free_pages[cnt] = table[b, j]
                    cnt += 1
                    table[b, j] = -1
            return new, cnt
        monkeypatch.setattr(kv, "crop_paged", bad)
        check = test_paged_hand_case
    else:
        def bad(caches, seq_len, n, appended, keep_extra, clear):   # clears one kept entry too
            return orig_c(caches, np.asarray(seq_len) - 1, n, appended + 1, keep_extra, clear) + 1
        monkeypatch.setattr(kv, "crop_contiguous", bad)
        check = test_contiguous_hand_case
    with pytest.raises(AssertionError):
        check()
