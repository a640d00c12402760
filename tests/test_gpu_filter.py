"""Top-k / top-p keep thresholds on the GPU (spec_filter_thresholds) against the
oracle's (oracle/adjust.py), row by row.

top-k thresholds must be equal exactly.  top-p thresholds must be equal except
in rows whose nucleus boundary lies within the derived band of top_p
(parity.nucleus_bands: the kernels' fp32 weights may put such a tie group on
either side).  The rows in the band are counted; the rows whose threshold
actually differs must all lie in it, and may be at most a twentieth of a
case's rows.  (Untied logits put about 1/V of the mass in each tie group, so
the worst-case fp32 band of a few 1e-6 covers a fair share of rows, while the
kernels' actual error is far smaller.)

Every case also runs with the workspace, where a top-k of at most 64 selects
from the chunks' candidate lists (rows of ties overflow the lists and take the
row path), and top-p alone takes the streaming nucleus path (rows it cannot
finish take the row path).  Both runs are held to the oracle on their own: the
two paths weigh tokens in different fp32 arithmetic, so in-band rows may
differ between them.

The cases reach every path of the threshold kernel: the register-resident
histogram and candidate list, the survivors-only nucleus after top-k, one
refinement level of a crossing bin too large for the list, the whole-row radix
select for rows longer than the registers hold, rows whose finite logits are
all equal, -inf entries and heavy ties.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import adjust
from tests import gpu_util, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_util.device()


def _banner(msg):
    print(f"[filter] {msg}", flush=True)


def _check(dev, target, draft, dtype, T, k, p, where):
    """target [B, G+1, V], draft [B, G, V] as float32 (bf16: already bf16-exact).
    Runs without and with the workspace (a top-k of at most 64 then selects
    from chunk candidate lists, top-p alone takes the nucleus path); each run's
    thresholds are checked against the oracle, and the workspace must come
    back zeroed."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    B, g1, V = target.shape
    if dtype == "bf16":
        tt = gpu_util.to_gpu(W.f32_to_bf16_bits(target), "bf16", dev)
        dd = gpu_util.to_gpu(W.f32_to_bf16_bits(draft), "bf16", dev)
    else:
        tt, dd = gpu_util.to_gpu(target, "f32", dev), gpu_util.to_gpu(draft, "f32", dev)
    _banner(f"{where}: B={B} gamma={g1 - 1} V={V} {dtype} T={T} top_k={k} top_p={p}")
    gt, gd = sv.filter_thresholds(tt, dd, T, k, p)
    got = np.concatenate([gt.cpu().numpy().ravel(), gd.cpu().numpy().ravel()])
    ws = torch.zeros(sv.filter_workspace_size(B, g1 - 1, V), dtype=torch.uint8, device=dev)
    lt, ld = sv.filter_thresholds(tt, dd, T, k, p, workspace=ws)
    got_l = np.concatenate([lt.cpu().numpy().ravel(), ld.cpu().numpy().ravel()])
    assert int(torch.count_nonzero(ws)) == 0, f"{where}: workspace not left zeroed"
    if 0 < k <= 64 and k < V:
        # the chunk lists pick the same keys with the same weights as the row path
        np.testing.assert_array_equal(got_l, got, err_msg=f"{where}: list path differs")
    rows = np.concatenate([target.reshape(-1, V), draft.reshape(-1, V)]).astype(np.float64)
    tau, margin = adjust.thresholds(rows, T, k, p)
    ok = margin > parity.nucleus_bands(rows, float(np.float32(T)), k)
    want = tau.astype(np.float32)
    for name, g in (("row path", got), ("workspace path", got_l)):
        differ = g != want
        bad = np.nonzero(ok & differ)[0]
        assert bad.size == 0, (f"{where} ({name}): rows {bad[:8]} thresholds {g[bad[:8]]} != oracle "
                               f"{want[bad[:8]]} (margins {margin[bad[:8]]})")
        for i in np.nonzero(differ)[0]:  # in the band: one tie group kept more or less at most
            near = parity.adjacent_values(rows[i], tau[i])
            assert g[i] in near, (f"{where} ({name}): row {i} threshold {g[i]} is not the oracle's {want[i]} "
                                  f"or an adjacent logit {near}")
        amb, ndiff = int((~ok).sum()), int(differ.sum())
        _banner(f"  {name}: rows={len(g)} in_band={amb} differ={ndiff}")
        assert ndiff <= max(1, len(g) // 20), f"{where} ({name}): {ndiff} of {len(g)} thresholds differ"


def _bf16(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32)))


@pytest.mark.parametrize("k,p", [(50, 1.0), (0, 0.9), (50, 0.9), (2000, 0.95), (60000, 1.0), (1, 0.5)])
def test_full_size_bf16_rows(dev, k, p):
    """The B=64, gamma=4, V=128256 bf16 workload's row recipe (4 sequences):
    Gaussian logits with 8 peaked tokens, many bf16 ties."""
    case = W.config3(7, 1.0, B=4)
    t = W.bf16_bits_to_f32(case.target)
    d = W.bf16_bits_to_f32(case.draft)
    _check(dev, t, d, "bf16", 1.0, k, p, "cfg3 rows")


@pytest.mark.parametrize("T", [0.5, 2.0])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gaussian_rows(dev, dt, T):
    case = W.gaussian_case(6, 3, 32128, "f32", T, seed=71, target_std=3.0)
    t, d = (case.target, case.draft) if dt == "f32" else (_bf16(case.target), _bf16(case.draft))
    for k, p in ((40, 0.8), (0, 0.95), (500, 1.0)):
        _check(dev, t, d, dt, T, k, p, f"gauss {dt}")


def test_crossing_bin_refined_once(dev):
    """N(0, 1) logits with one token at +50 and one at -50: the 16 bins over
    [-50, 50] are 6.25 wide, so the body of the row (all 128254 other tokens)
    falls in two bins, more than the 32768-entry list; one level of 16 finer
    bins splits it.  top-k near the median and top-p at T = 8 (nearly flat
    weights) both cross inside it."""
    rng = np.random.default_rng(72)
    V = 128256
    x = rng.standard_normal((2, 2, V)).astype(np.float32)
    x[..., 10] = 50.0
    x[..., 20] = -50.0
    x = _bf16(x)
    t, d = x[:, :2], x[:, :1]
    _check(dev, t, d, "bf16", 8.0, 64000, 1.0, "refined top-k")
    _check(dev, t, d, "bf16", 8.0, 0, 0.5, "refined top-p")
    _check(dev, t, d, "bf16", 8.0, 90000, 0.7, "refined both")


def test_refinement_overflow_takes_the_row_radix_select(dev):
    """bf16 rows of 131072 tokens (the register capacity) with outliers at
    +-10^4: the body stays in one bin even at the finer level (78 logits wide),
    so the row falls back to the radix select from memory."""
    rng = np.random.default_rng(73)
    V = 131072
    x = rng.standard_normal((1, 2, V)).astype(np.float32)
    x[..., 3] = 1e4
    x[..., 4] = -1e4
    x = _bf16(x)
    _check(dev, x[:, :2], x[:, :1], "bf16", 1.0, 70000, 1.0, "overflow top-k")
    _check(dev, x[:, :2], x[:, :1], "bf16", 1000.0, 0, 0.6, "overflow top-p")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unaligned_rows(dev, dt):
    """V = 50257: rows that are not 16-byte aligned take element loads."""
    case = W.gaussian_case(3, 2, 50257, "f32", 1.0, seed=78, target_std=3.0)
    t, d = (case.target, case.draft) if dt == "f32" else (_bf16(case.target), _bf16(case.draft))
    for k, p in ((40, 1.0), (0, 0.9), (300, 0.7)):
        _check(dev, t, d, dt, 1.0, k, p, f"unaligned {dt}")


def test_rows_longer_than_the_registers(dev):
    """fp32 rows of 70000 tokens exceed the 65536 the registers hold."""
    case = W.gaussian_case(2, 2, 70000, "f32", 1.0, seed=74, target_std=2.0)
    # (30, .): the chunk lists decide these rows without holding them
    for k, p in ((100, 1.0), (0, 0.9), (100, 0.9), (30, 1.0), (30, 0.9)):
        _check(dev, case.target, case.draft, "f32", 1.0, k, p, "long f32")


def test_constant_rows_neg_inf_and_ties(dev):
    rng = np.random.default_rng(75)
    V = 4096
    t = rng.integers(-3, 4, size=(4, 3, V)).astype(np.float32)   # 7 values: every row is tie groups
    t[0, 0] = 1.5                                                 # all equal
    t[1, 1] = -np.inf
    t[1, 1, :7] = np.arange(7, dtype=np.float32)                  # 7 finite values, the rest -inf
    t[2, 2, ::2] = -np.inf                                        # half -inf
    d = t[:, :2].copy()
    for k, p in ((1, 1.0), (5, 1.0), (10, 1.0), (3000, 1.0), (0, 0.3), (0, 0.99), (20, 0.6)):
        _check(dev, t, d, "f32", 1.0, k, p, f"ties k={k} p={p}")


def test_small_rows_and_extreme_k(dev):
    case = W.gaussian_case(3, 2, 64, "f32", 1.0, seed=76)
    for k, p in ((63, 1.0), (1, 1.0), (32, 0.999), (0, 0.001)):
        _check(dev, case.target, case.draft, "f32", 1.0, k, p, f"V=64 k={k} p={p}")


def test_no_active_filter_keeps_every_row(dev):
    case = W.gaussian_case(2, 2, 256, "f32", 1.0, seed=77)
    import speculative_sampling_verification_02_amd as sv
    tt, dd = gpu_util.to_gpu(case.target, "f32", dev), gpu_util.to_gpu(case.draft, "f32", dev)
    for k, p in ((0, 1.0), (256, 1.0), (-3, 1.5)):
        gt, gd = sv.filter_thresholds(tt, dd, 1.0, k, p)
        assert np.all(np.isneginf(gt.cpu().numpy())) and np.all(np.isneginf(gd.cpu().numpy()))


@pytest.mark.parametrize("k", [1, 4, 63, 64, 65])
def test_list_path_boundaries(dev, k):
    """top-k at and around the largest k the chunk lists take (64), on the
    B=64 workload's row recipe (2 sequences), with and without top-p."""
    case = W.config3(9, 1.0, B=2)
    t = W.bf16_bits_to_f32(case.target)
    d = W.bf16_bits_to_f32(case.draft)
    for p in (1.0, 0.8):
        _check(dev, t, d, "bf16", 1.0, k, p, f"list k={k}")


def test_list_path_with_one_overflowing_chunk(dev):
    """Rows whose second 8192-token chunk is one repeated value next to rows
    whose lists all fit.  Every value of such a chunk is at or above its pivot,
    so its list overflows and the row takes the row path; the other rows take
    the lists, in the same launch."""
    rng = np.random.default_rng(79)
    V = 40000
    x = rng.standard_normal((3, 3, V)).astype(np.float32) * 2.0
    x[0, 1, 8192:16384] = 7.5            # above the rest of the row: the top-k is one tie group
    x[1, 0, 8192:16384] = -1.0           # inside the body of the row
    x = _bf16(x)
    for k, p in ((10, 1.0), (50, 0.9), (64, 1.0)):
        _check(dev, x, x[:, :2].copy(), "bf16", 1.0, k, p, f"overflow chunk k={k}")


def test_list_path_unaligned_f32(dev):
    case = W.gaussian_case(2, 2, 20011, "f32", 1.0, seed=80, target_std=3.0)
    for k, p in ((7, 1.0), (40, 0.7)):
        _check(dev, case.target, case.draft, "f32", 1.0, k, p, f"unaligned f32 k={k}")


def test_nucleus_path_crossing_in_a_tail_bin(dev):
    """One token 27 logits above an N(0, 1) body at T = 1 (39 octaves) and
    top_p = 1 - 1.2e-7 (the body holds 2e-7 of the mass): the crossing lies in
    the body, more than 31 octaves below the top of the spike's chunk, inside
    that chunk's tail bin.  The nucleus path leaves such a row to the row path;
    the rows without a spike (their crossing deep in the body's lower tail) it
    finishes itself."""
    rng = np.random.default_rng(81)
    V = 65536
    x = rng.standard_normal((2, 2, V)).astype(np.float32)
    x[0, 0, 100] = 27.0
    x[1, 1, 40000] = 27.0
    x = _bf16(x)
    _check(dev, x, x[:, :1].copy(), "bf16", 1.0, 0, float(np.float32(0.9999999)), "tail crossing")


def test_nucleus_rows_listing_more_than_the_pick_holds(dev):
    """fp32 rows of 270000 tokens (33 chunks of 8192) of N(0, 2.5) logits: at
    top_p 0.9 the crossing octave holds about 14000 logits, more than the pick
    kernel gathers (8192), so those rows go to the row kernel and the pick
    kernel must still clear every listed entry (the workspace comes back
    zeroed)."""
    case = W.gaussian_case(2, 1, 270000, "f32", 1.0, seed=82, target_std=2.5)
    for p in (0.9, 0.5):
        _check(dev, case.target, case.draft, "f32", 1.0, 0, p, f"33 chunks p={p}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_nucleus_rows_near_the_band(dev, dt):
    """The top-p rows of the filtered verification tests (V = 20008, N(0, 2.5)
    logits, top_p 0.9): several rows' nucleus boundaries lie within the band,
    where the row kernel and the streaming launches may keep a tie group more
    or less; each is held to the oracle on its own."""
    case = W.gaussian_case(8, 4, 20008, dt, 1.0, seed=47, target_std=2.5, draft_noise=1.0)
    if dt == "bf16":
        t, d = W.bf16_bits_to_f32(case.target), W.bf16_bits_to_f32(case.draft)
    else:
        t, d = case.target, case.draft
    _check(dev, t, d, dt, 1.0, 0, 0.9, f"near-band rows {dt}")
