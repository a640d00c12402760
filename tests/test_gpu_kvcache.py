"""GPU parity of the KV-cache crop (spec_kv_crop, spec_kv_crop_paged) against
the slicing oracle (oracle/kvcache.py), bit for bit: cache bytes, lengths,
block tables and the free list.

The crop is queued right after a real verification on the same stream with no
synchronisation in between, so it reads n_accepted on the device as a serving
loop would; the oracle gets the n_accepted that verification produced.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import kvcache as okv
from tests import gpu_util

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_util.device()


def _verify_then(case, dev, crop):
    """Launch the verification, then crop(n_accepted_tensor), with no sync."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    t = gpu_util.case_tensors(case, dev)
    out = sv.verify(t["target"], t["draft"], t["tokens"], t["uniforms"], case.temperature)
    crop(out["n_accepted"])
    torch.cuda.synchronize(dev)
    return out["n_accepted"].cpu().numpy()


@pytest.mark.parametrize("appended,keep_extra,clear,T", [(4, 0, True, 1.0), (5, 1, True, 1.0), (4, 0, False, 1.0),
                                                         (5, 1, True, 0.0)])
def test_contiguous_crop_after_verify(dev, appended, keep_extra, clear, T):
    import torch
    import speculative_sampling_verification_02_amd as sv
    B, G, H, S_max, D = 64, 4, 8, 96, 128
    case = W.config3(20, T, B=B, V=16384)
    rng = np.random.default_rng(21)
    caches = [torch.from_numpy(rng.integers(1, 2 ** 15, size=(B, H, S_max, D)).astype(np.int16)).to(dev)
              .view(torch.bfloat16) for _ in range(6)]
    seq_np = rng.integers(0, S_max - appended + 3, size=B).astype(np.int32)   # a few write past S_max
    seq_len = torch.from_numpy(seq_np).to(dev)
    host = [c.view(torch.int16).cpu().numpy() for c in caches]
    print(f"[kv] contiguous B={B} H={H} S_max={S_max} D={D} x{len(caches)} appended={appended} "
          f"keep_extra={keep_extra} clear={clear} T={T}", flush=True)
    n = _verify_then(case, dev, lambda n_acc: sv.kv_crop(caches, seq_len, n_acc, appended, keep_extra, clear))
    want_len = okv.crop_contiguous(host, seq_np, n, appended, keep_extra, clear)
    assert np.array_equal(seq_len.cpu().numpy(), want_len)
    for c, h in zip(caches, host):
        assert np.array_equal(c.view(torch.int16).cpu().numpy(), h)


def test_contiguous_crop_leaves_failed_sequences(dev):
    import torch
    import speculative_sampling_verification_02_amd as sv
    B, H, S_max, D = 40, 2, 16, 8
    rng = np.random.default_rng(22)
    cache = torch.from_numpy(rng.random((B, H, S_max, D), dtype=np.float32) + 1).to(dev)
    host = cache.cpu().numpy()
    seq_np = rng.integers(0, 12, size=B).astype(np.int32)
    n_np = rng.integers(-1, 5, size=B).astype(np.int32)          # -1: a sequence with no result
    seq_len, n_acc = torch.from_numpy(seq_np).to(dev), torch.from_numpy(n_np).to(dev)
    sv.kv_crop([cache], seq_len, n_acc, 4, 0, True)
    torch.cuda.synchronize(dev)
    want = okv.crop_contiguous([host], seq_np, n_np, 4, 0, True)
    assert np.array_equal(seq_len.cpu().numpy(), want)
    assert np.array_equal(cache.cpu().numpy(), host)


def _paged_state(rng, B, max_blocks, P, num_pages, seq_np, appended):
    table = np.full((B, max_blocks), -1, np.int32)
    ids = rng.permutation(num_pages).astype(np.int32)
    k = 0
    for b in range(B):
        for j in range(min(max_blocks, -(-(int(seq_np[b]) + appended) // P))):
            table[b, j] = ids[k]
            k += 1
    free = np.full(num_pages, -7, np.int32)
    free[:num_pages - k] = ids[k:]
    return table, free, num_pages - k


@pytest.mark.parametrize("appended,keep_extra,clear,P", [(4, 0, True, 16), (5, 1, True, 4), (4, 0, False, 16),
                                                         (9, 0, True, 1)])
def test_paged_crop_after_verify(dev, appended, keep_extra, clear, P):
    import torch
    import speculative_sampling_verification_02_amd as sv
    B, G, H, D, max_blocks = 64, 4, 8, 128, 40
    case = W.config3(23, 1.0, B=B, V=16384)
    rng = np.random.default_rng(24)
    seq_np = rng.integers(0, (max_blocks - 2) * P - appended, size=B).astype(np.int32)
    num_pages = B * max_blocks + 17
    table_np, free_np, count = _paged_state(rng, B, max_blocks, P, num_pages, seq_np, appended)
    caches = [torch.from_numpy(rng.integers(1, 2 ** 15, size=(num_pages, P, H, D)).astype(np.int16)).to(dev)
              for _ in range(2)]
    host = [c.cpu().numpy() for c in caches]
    table, seq_len = torch.from_numpy(table_np.copy()).to(dev), torch.from_numpy(seq_np).to(dev)
    free, fcount = torch.from_numpy(free_np.copy()).to(dev), torch.tensor([count], dtype=torch.int32, device=dev)
    print(f"[kv] paged B={B} pages={num_pages} page_size={P} appended={appended} keep_extra={keep_extra} "
          f"clear={clear}", flush=True)
    n = _verify_then(case, dev, lambda n_acc: sv.kv_crop_paged(caches, table, seq_len, n_acc, appended, free, fcount,
                                                               keep_extra, clear))
    want_len, want_count = okv.crop_paged(host, table_np, seq_np, n, appended, keep_extra, clear, free_np, count,
                                          P, num_pages)
    assert np.array_equal(seq_len.cpu().numpy(), want_len)
    assert np.array_equal(table.cpu().numpy(), table_np)
    assert int(fcount.item()) == want_count
    assert np.array_equal(free.cpu().numpy(), free_np)
    for c, h in zip(caches, host):
        assert np.array_equal(c.cpu().numpy(), h)


def test_paged_crop_many_sequences_without_clear(dev):
    """More sequences than the finishing workgroup's threads (the release
    carries its count across chunks of 1024), no caches, some -1 results."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    B, max_blocks, P, appended = 2500, 3, 8, 6
    rng = np.random.default_rng(25)
    seq_np = rng.integers(0, 2 * P - appended, size=B).astype(np.int32)
    num_pages = B * max_blocks
    table_np, free_np, count = _paged_state(rng, B, max_blocks, P, num_pages, seq_np, appended)
    n_np = rng.integers(-1, appended + 1, size=B).astype(np.int32)
    table, seq_len = torch.from_numpy(table_np.copy()).to(dev), torch.from_numpy(seq_np).to(dev)
    free, fcount = torch.from_numpy(free_np.copy()).to(dev), torch.tensor([count], dtype=torch.int32, device=dev)
    sv.kv_crop_paged([], table, seq_len, torch.from_numpy(n_np).to(dev), appended, free, fcount, 0, False,
                     page_size=P, num_pages=num_pages)
    torch.cuda.synchronize(dev)
    want_len, want_count = okv.crop_paged([], table_np, seq_np, n_np, appended, 0, False, free_np, count, P,
                                          num_pages)
    assert np.array_equal(seq_len.cpu().numpy(), want_len)
    assert np.array_equal(table.cpu().numpy(), table_np)
    assert int(fcount.item()) == want_count
    assert np.array_equal(free.cpu().numpy(), free_np)
