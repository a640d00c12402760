"""Bounded cross-workgroup waits and their give-up path, forced from the host.

spec_set_wait_limit(1) makes every cross-workgroup wait of the next launch give
up unless its data is already there at the first poll: the fused path's waits,
and at temperature 0 the waits of the multipass path's finishing workgroups on
the per-chunk argmax words.  Sequences then lose their result while every
kernel still runs to its end.  The contract (include/specverify.h): a sequence whose wait gave up
reports n_accepted = next_token = -1, every other sequence has its full
result, and the workspace must be zero-filled again before its next use; after
that the next call is whole again.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_util, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_util.device()


@pytest.mark.parametrize("T,dt,polls", [(1.0, "bf16", 1), (0.0, "bf16", 1), (1.0, "f32", 1),
                                         (1.0, "bf16", 2), (1.0, "bf16", 4), (1.0, "bf16", 8), (0.0, "bf16", 4),
                                         (1.0, "bf16", 16), (1.0, "bf16", 64)])
def test_waits_that_give_up_report_minus_one(dev, T, dt, polls):
    """One poll per wait: every wait whose data is late gives up (nearly every
    sequence).  A few polls on the B=64, V=128256 batch: the sequences whose
    items come first can finish while later ones give up -- in every case each
    sequence is -1 or the oracle's result."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    case = W.config3(90, T, B=64) if polls > 1 else W.gaussian_case(24, 4, 40000, dt, T, seed=90, target_std=2.5)
    ws = torch.zeros(sv.workspace_size(case.B, case.gamma, case.V, sv.SPEC_BF16), dtype=torch.uint8, device=dev)
    t = gpu_util.case_tensors(case, dev)
    print(f"[giveup] B={case.B} gamma={case.gamma} V={case.V} {case.dtype} T={T}, {polls} poll(s) per wait",
          flush=True)
    sv.set_wait_limit(polls)
    try:
        out = gpu_util.run_case(case, sv.ALGO_FUSED, tensors=t, dev=dev, workspace=ws)
    finally:
        sv.set_wait_limit(0)
    n, tok = out["n_accepted"], out["next_token"]
    lost = n == -1
    print(f"[giveup] {int(lost.sum())} of {case.B} sequences gave up", flush=True)
    if polls == 1:
        assert lost.any(), "with one poll per wait some wait must find its data late"
    assert np.array_equal(tok == -1, lost)
    kept = np.nonzero(~lost)[0]
    if kept.size:
        parity.check(case, out, seqs=kept, where="the sequences that did not give up")
    # recovery as documented: zero the workspace; the next call is whole again
    ws.zero_()
    again = gpu_util.run_case(case, sv.ALGO_FUSED, tensors=t, dev=dev, workspace=ws)
    assert (again["n_accepted"] >= 0).all()
    parity.check(case, again, where="after re-zeroing")
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("polls,B", [(1, 24), (1, 64), (4, 64)])
def test_multipass_argmax_waits_that_give_up_report_minus_one(dev, polls, B):
    """The multipass path at temperature 0: its finishing workgroups are the
    last of the grid and may find some chunk words still unpublished.  Whether
    any wait gives up depends on the dispatch order, so only the contract is
    checked: each sequence is -1 (both outputs) or the oracle's result, and a
    re-zeroed workspace gives the whole result again."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    case = W.config3(91, 0.0, B=B) if B == 64 else W.gaussian_case(B, 4, 40000, "bf16", 0.0, seed=91,
                                                                   target_std=2.5)
    ws = torch.zeros(sv.workspace_size(case.B, case.gamma, case.V, sv.SPEC_BF16), dtype=torch.uint8, device=dev)
    t = gpu_util.case_tensors(case, dev)
    print(f"[giveup] multipass B={case.B} gamma={case.gamma} V={case.V} T=0, {polls} poll(s) per wait",
          flush=True)
    sv.set_wait_limit(polls)
    try:
        out = gpu_util.run_case(case, sv.ALGO_MULTIPASS, tensors=t, dev=dev, workspace=ws)
    finally:
        sv.set_wait_limit(0)
    n, tok = out["n_accepted"], out["next_token"]
    lost = n == -1
    print(f"[giveup] {int(lost.sum())} of {case.B} sequences gave up", flush=True)
    assert np.array_equal(tok == -1, lost)
    kept = np.nonzero(~lost)[0]
    if kept.size:
        parity.check(case, out, seqs=kept, where="the sequences that did not give up")
    if not lost.any():
        assert int(ws.count_nonzero()) == 0
    ws.zero_()
    again = gpu_util.run_case(case, sv.ALGO_MULTIPASS, tensors=t, dev=dev, workspace=ws)
    assert (again["n_accepted"] >= 0).all()
    parity.check(case, again, where="after re-zeroing")
    assert int(ws.count_nonzero()) == 0
