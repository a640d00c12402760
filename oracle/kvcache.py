"""KV-cache crop after a verification step, as plain slicing.

TEST INFRASTRUCTURE, like the rest of oracle/.  Page abbreviations are listed
in oracle/__init__.py.

[FI] "The loop: draft, verify in one pass, keep a prefix" (the paragraph on
the KV cache): the verification pass appends the drafts' entries to the
target's cache, and after the accept test the entries beyond the accepted
prefix are discarded, so that the next step starts from exactly the tokens
that were emitted -- one crop call after the sampling function.  [LH] "Fix the
benchmark conditions first": the target cache must follow the committed
prefix and deal with the state of rejected drafts; with paged storage that
state is whole pages, returned to the pool.

Readings taken where the pages are silent (each is listed in the design notes):
  * seq_len[b] on entry is the committed length before the verification pass;
    the pass wrote entries seq_len[b] .. seq_len[b] + appended - 1.  The crop
    keeps keep_extra of those plus one per accepted draft: the new length is
    seq_len[b] + keep_extra + n_accepted[b].  (keep_extra = 1 when the pass
    also wrote the entry of the previous step's final token.)  The final token
    of this step is not in the cache; the next pass writes it.
  * "Discarded" entries are zero-filled when `clear` is set; without it only
    the length changes.  Entries at or past the cache's capacity are never
    touched.
  * Paged storage: page j of a sequence holds its positions j*P .. j*P + P - 1
    (P = page_size), at block_table[b][j] (-1: no page).  Every page of the
    sequence at block index >= ceil(new_len / P) is released: its id is
    appended to the free list (sequences in order, blocks in ascending order)
    and its table entry becomes -1.
  * A sequence whose verification reported n_accepted = -1 (no result) is
    left as it was.
"""

from __future__ import annotations

import numpy as np


def crop_contiguous(caches, seq_len, n_accepted, appended: int, keep_extra: int, clear: bool):
    """caches: arrays [B][H][S_max][D] (modified in place); seq_len: int [B]
    (returned updated, the input untouched).  Positions below 0 or at or past
    S_max are never touched."""
    seq_len = np.asarray(seq_len, dtype=np.int64)
    out_len = seq_len.copy()
    for b in range(len(seq_len)):
        n = int(n_accepted[b])
        if n < 0:
            continue
        new_len = int(seq_len[b]) + keep_extra + n
        written_end = int(seq_len[b]) + appended
        if clear:
            for cache in caches:
                s_max = cache.shape[2]
                lo = min(max(new_len, 0), s_max)
                hi = min(max(written_end, 0), s_max)
                if lo < hi:
                    cache[b, :, lo:hi, :] = 0
        out_len[b] = new_len
    return out_len


def crop_paged(caches, block_table, seq_len, n_accepted, appended: int, keep_extra: int, clear: bool,
               free_pages, free_count: int, page_size: int, num_pages: int):
    """caches: arrays [num_pages][page_size][H][D] (modified in place; none
    are needed without `clear`); block_table: int [B][max_blocks]
    (modified in place; an entry outside [0, num_pages) names no page of these
    caches); free_pages: int array with room for every page (modified in place
    from free_count on).  Lengths below 0 count as 0.  Returns (new seq_len,
    new free_count)."""
    seq_len = np.asarray(seq_len, dtype=np.int64)
    out_len = seq_len.copy()
    B, max_blocks = block_table.shape
    for b in range(B):
        n = int(n_accepted[b])
        if n < 0:
            continue
        new_len = int(seq_len[b]) + keep_extra + n
        written_end = int(seq_len[b]) + appended
        if clear:
            for s in range(max(new_len, 0), written_end):
                j = s // page_size
                if j >= max_blocks or not 0 <= block_table[b, j] < num_pages:
                    continue
                for cache in caches:
                    cache[block_table[b, j], s % page_size] = 0
        first_free = -(-max(new_len, 0) // page_size)
        for j in range(first_free, max_blocks):
            if block_table[b, j] >= 0:
                free_pages[free_count] = block_table[b, j]
                free_count += 1
                block_table[b, j] = -1
        out_len[b] = new_len
    return out_len, free_count
