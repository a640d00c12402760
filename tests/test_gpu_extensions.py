"""GPU parity of the two extensions of spec_verify_ex -- the lenience factor and
per-sequence draft counts -- through the C ABI, against the fp64 oracle with the
same settings (rules in tests/parity.py)."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_util, parity

pytestmark = pytest.mark.gpu

ALGOS = {"multipass": 1, "fused": 2}


@pytest.fixture(scope="module")
def dev():
    return gpu_util.device()


def _banner(msg):
    print(f"[ext] {msg}", flush=True)


def _gseq(rng, B, G):
    g = rng.integers(0, G + 1, size=B)
    g[0], g[-1] = 0, G          # always one plain decoding step and one full draft
    return g


@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1.0, 0.6, 0.0])
@pytest.mark.parametrize("l", [0.5, 0.1])
def test_lenience(dev, algo, dt, T, l):
    case = W.gaussian_case(12, 5, 20008, dt, T, seed=41, target_std=2.5, draft_noise=1.5)
    _banner(f"lenience {algo} {dt} T={T} l={l}")
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, lenience=l)
    rep = parity.check(case, gpu, where=f"lenience {dt} T{T} l{l}", lenience=l)
    _banner(f"  {rep}")


@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_ragged_gamma(dev, algo, dt, T):
    rng = np.random.default_rng(42)
    case = W.gaussian_case(16, 6, 20008, dt, T, seed=42, target_std=2.0, draft_noise=0.7)
    g = _gseq(rng, case.B, case.gamma)
    _banner(f"ragged {algo} {dt} T={T} gamma_b={g.tolist()}")
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, gamma_seq=g)
    rep = parity.check(case, gpu, where=f"ragged {dt} T{T}", gamma_seq=g)
    assert np.all(gpu["n_accepted"] <= g)
    _banner(f"  {rep}")


@pytest.mark.parametrize("B", [2048, 2049])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_ragged_batch_at_the_fused_limit(dev, B, T):
    """The fused kernels keep every sequence's draft count in LDS for batches of
    up to 2048 sequences (32 chunks of 64, the last chunk full at 2048) and
    decline larger ones with draft counts, which the automatic choice then
    runs on the multipass path."""
    import speculative_sampling_verification_02_amd as sv
    rng = np.random.default_rng(B)
    case = W.gaussian_case(B, 3, 136, "bf16", T, seed=B, target_std=2.0, draft_noise=0.7)
    g = _gseq(rng, case.B, case.gamma)
    _banner(f"ragged batch B={B} T={T} live pairs={int(g.sum())}")
    if B > 2048:
        t = gpu_util.case_tensors(case, dev)
        gs = __import__("torch").from_numpy(g.astype(np.int32)).to(dev)
        with pytest.raises(sv.SpecVerifyError) as e:
            sv.verify(t["target"], t["draft"], t["tokens"], t["uniforms"], T, algo=sv.ALGO_FUSED, gamma_seq=gs)
        assert e.value.status == sv.SPEC_EUNSUPPORTED
    algo = sv.ALGO_FUSED if B <= 2048 else sv.ALGO_AUTO
    gpu = gpu_util.run_case(case, algo, dev=dev, gamma_seq=g)
    rep = parity.check(case, gpu, where=f"ragged B={B} T{T}", gamma_seq=g)
    assert np.all(gpu["n_accepted"] <= g)
    _banner(f"  {rep}")


@pytest.mark.parametrize("T", [1.0, 0.8])
def test_long_walk_odd_batch_with_every_extension(dev, T):
    """An odd batch with about ten pairs per team (85 * 5 over 42 teams), with
    draft counts, lenience and a nucleus filter at once."""
    rng = np.random.default_rng(85)
    case = W.gaussian_case(85, 5, 128256, "bf16", T, seed=85, target_std=2.5, draft_noise=0.8)
    g = _gseq(rng, case.B, case.gamma)
    gpu = gpu_util.run_case(case, ALGOS["fused"], dev=dev, gamma_seq=g, lenience=0.8, top_p=0.9)
    thr = gpu_util.gpu_thresholds(case, 0, 0.9, dev=dev)
    rep = parity.check(case, gpu, where=f"bonus units ext T{T}", gamma_seq=g, lenience=0.8, top_p=0.9,
                       gpu_thresholds=thr, workers=8)
    assert np.all(gpu["n_accepted"] <= g)
    _banner(f"  {rep}")
    assert rep.thresholds_differ <= 2
    assert rep.token_mismatch_valid <= 2


@pytest.mark.parametrize("algo", list(ALGOS))
def test_ragged_and_lenient_together(dev, algo):
    rng = np.random.default_rng(43)
    case = W.gaussian_case(20, 4, 9000, "bf16", 1.0, seed=43, target_std=2.0, draft_noise=1.2)
    g = _gseq(rng, case.B, case.gamma)
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, gamma_seq=g, lenience=0.3)
    rep = parity.check(case, gpu, where="ragged+lenient", gamma_seq=g, lenience=0.3)
    _banner(f"ragged+lenient {algo}: {rep}")


@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_full_size_ragged_lenient(dev, algo, T):
    """The B=64, gamma=4, V=128256 bf16 workload in the launch configuration the
    bench times, with random per-sequence draft counts and l = 0.5."""
    rng = np.random.default_rng(44)
    case = W.config3(2, T)
    g = _gseq(rng, case.B, case.gamma)
    _banner(f"full size ragged lenient {algo} T={T}")
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, gamma_seq=g, lenience=0.5)
    rep = parity.check(case, gpu, where=f"cfg3 ragged lenient T{T}", gamma_seq=g, lenience=0.5)
    _banner(f"  {rep}")
    assert rep.token_mismatch_valid <= max(1, case.B // 20)


@pytest.mark.parametrize("algo", list(ALGOS))
def test_out_of_range_counts_are_clamped_and_workspace_stays_zero(dev, algo):
    import torch
    import speculative_sampling_verification_02_amd as sv
    case = W.gaussian_case(6, 3, 4096, "f32", 1.0, seed=45)
    ws = torch.zeros(sv.workspace_size(case.B, case.gamma, case.V, sv.SPEC_F32), dtype=torch.uint8, device=dev)
    raw = np.array([-3, 0, 2, 3, 9, 1])
    clamped = np.clip(raw, 0, case.gamma)
    a = gpu_util.run_case(case, ALGOS[algo], dev=dev, gamma_seq=raw, workspace=ws)
    assert int(ws.count_nonzero()) == 0
    b = gpu_util.run_case(case, ALGOS[algo], dev=dev, gamma_seq=clamped, workspace=ws)
    assert int(ws.count_nonzero()) == 0
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    parity.check(case, b, where="clamped", gamma_seq=clamped)


def test_bad_lenience_is_rejected(dev):
    import torch
    import speculative_sampling_verification_02_amd as sv
    case = W.gaussian_case(2, 2, 512, "f32", 1.0, seed=46)
    t = gpu_util.case_tensors(case, dev)
    for l in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(sv.SpecVerifyError) as e:
            sv.verify(t["target"], t["draft"], t["tokens"], t["uniforms"], 1.0, lenience=l)
        assert e.value.status == sv.SPEC_EINVAL
    torch.cuda.synchronize(dev)


# ------------------------------------------------------------ top-k / top-p

@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k,p", [(50, 1.0), (0, 0.9), (200, 0.8), (1, 1.0), (3000, 0.5), (0, 0.2)])
def test_topk_topp(dev, dt, k, p, algo):
    case = W.gaussian_case(8, 4, 20008, dt, 1.0, seed=47, target_std=2.5, draft_noise=1.0)
    _banner(f"filter {dt} top_k={k} top_p={p} {algo}")
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, top_k=k, top_p=p)
    thr = gpu_util.gpu_thresholds(case, k, p, dev=dev)
    rep = parity.check(case, gpu, where=f"filter {dt} k{k} p{p}", top_k=k, top_p=p, gpu_thresholds=thr)
    _banner(f"  {rep}")
    assert rep.thresholds_differ <= 1
    assert rep.token_mismatch_valid <= 1


@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k,p", [(64, 1.0), (0, 0.9)])
def test_topk_topp_long_rows(dev, dt, k, p, algo):
    """Rows of 160000 tokens (80 wave tiles, more than 64): the fused kernel's
    wide team wait, with keep thresholds."""
    case = W.gaussian_case(4, 3, 160000, dt, 1.0, seed=49, target_std=2.5, draft_noise=1.0)
    _banner(f"long-row filter {dt} top_k={k} top_p={p} {algo}")
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, top_k=k, top_p=p)
    thr = gpu_util.gpu_thresholds(case, k, p, dev=dev)
    rep = parity.check(case, gpu, where=f"long-row filter {dt} k{k} p{p}", top_k=k, top_p=p, gpu_thresholds=thr)
    _banner(f"  {rep}")
    assert rep.thresholds_differ <= 1
    assert rep.token_mismatch_valid <= 1


@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("T", [1.0, 0.5])
def test_full_size_filtered_with_every_extension(dev, T, algo):
    """The B=64, gamma=4, V=128256 bf16 workload (many bf16 ties) with top-k 64,
    top-p 0.9, lenience 0.7 and random per-sequence draft counts at once."""
    rng = np.random.default_rng(48)
    case = W.config3(3, T)
    g = _gseq(rng, case.B, case.gamma)
    _banner(f"full size filtered T={T}")
    gpu = gpu_util.run_case(case, ALGOS[algo], dev=dev, top_k=64, top_p=0.9, lenience=0.7, gamma_seq=g)
    thr = gpu_util.gpu_thresholds(case, 64, 0.9, dev=dev)
    rep = parity.check(case, gpu, where=f"cfg3 filtered T{T}", top_k=64, top_p=0.9, lenience=0.7, gamma_seq=g,
                       gpu_thresholds=thr, workers=8)
    _banner(f"  {rep}")
    assert rep.thresholds_differ <= 2
    assert rep.token_mismatch_valid <= 2


def test_filters_leave_argmax_mode_alone_and_workspace_zero(dev):
    import torch
    import speculative_sampling_verification_02_amd as sv
    case = W.gaussian_case(6, 3, 8192, "bf16", 0.0, seed=49)
    ws = torch.zeros(sv.workspace_size(case.B, case.gamma, case.V, sv.SPEC_BF16), dtype=torch.uint8, device=dev)
    a = gpu_util.run_case(case, ALGOS["fused"], dev=dev, workspace=ws)
    b = gpu_util.run_case(case, ALGOS["fused"], dev=dev, workspace=ws, top_k=5, top_p=0.3)
    for key in a:
        assert np.array_equal(a[key], b[key], equal_nan=True), key
    case1 = W.gaussian_case(6, 3, 8192, "bf16", 1.0, seed=49)
    gpu_util.run_case(case1, ALGOS["fused"], dev=dev, workspace=ws, top_k=5, top_p=0.3)
    assert int(ws.count_nonzero()) == 0


# (fp32 rows with V % 4 != 0 are declined by the fused path: test_gpu_parity.test_shapes)
@pytest.mark.parametrize("dt,algo", [("f32", "auto"), ("f32", "multipass"), ("bf16", "auto"), ("bf16", "multipass"),
                                     ("bf16", "fused")])
def test_filters_on_unaligned_rows(dev, dt, algo):
    """V = 50257 (an odd vocabulary): the rows do not all start on 16 bytes.
    In bf16 the extended fused kernel copies each row from its aligned-down
    start (and the default algorithm takes it); in fp32 the fused path
    declines and the default algorithm runs the multipass path.  The
    thresholds take element loads.  Every extension at once, workspace left
    zero."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    rng = np.random.default_rng(51)
    case = W.gaussian_case(6, 3, 50257, dt, 1.0, seed=51, target_std=2.5)
    g = _gseq(rng, case.B, case.gamma)
    ws = torch.zeros(sv.workspace_size(case.B, case.gamma, case.V, sv.SPEC_BF16 if dt == "bf16" else sv.SPEC_F32),
                     dtype=torch.uint8, device=dev)
    _banner(f"unaligned {dt} filters")
    algo_code = {"auto": 0, "multipass": ALGOS["multipass"], "fused": ALGOS["fused"]}[algo]
    gpu = gpu_util.run_case(case, algo_code, dev=dev, top_k=100, top_p=0.8, lenience=0.8, gamma_seq=g, workspace=ws)
    thr = gpu_util.gpu_thresholds(case, 100, 0.8, dev=dev)
    rep = parity.check(case, gpu, where=f"unaligned {dt}", top_k=100, top_p=0.8, lenience=0.8, gamma_seq=g,
                       gpu_thresholds=thr)
    _banner(f"  {rep}")
    assert rep.thresholds_differ <= 1
    assert rep.token_mismatch_valid <= 1
    assert int(ws.count_nonzero()) == 0


def test_bad_top_p_is_rejected(dev):
    import speculative_sampling_verification_02_amd as sv
    case = W.gaussian_case(2, 2, 1024, "f32", 1.0, seed=50)
    t = gpu_util.case_tensors(case, dev)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.verify(t["target"], t["draft"], t["tokens"], t["uniforms"], 1.0, top_p=0.0)
    assert e.value.status == sv.SPEC_EINVAL
