"""spec_verify_noalloc against spec_verify, through the C ABI.

The allocation-free entry point runs the same kernels on the library's own
per-device scratch array, so for the same inputs its outputs must equal
spec_verify's (with a zeroed workspace) bit for bit; which is also the parity
bar, since spec_verify is held to the oracle elsewhere.  Two calls in a row,
the second with a smaller input, check that the array is left zero by a
completed call and serves the next shape; a call with B == 0 clears it.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_util, parity

pytestmark = pytest.mark.gpu


def _outputs(torch, B, G, dev):
    return {"n_accepted": torch.empty(B, dtype=torch.int32, device=dev),
            "next_token": torch.empty(B, dtype=torch.int32, device=dev),
            "alpha": torch.empty(B, G, dtype=torch.float32, device=dev),
            "p_draft": torch.empty(B, G, dtype=torch.float32, device=dev),
            "q_draft": torch.empty(B, G, dtype=torch.float32, device=dev)}


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_noalloc_matches_spec_verify_on_two_calls(T):
    import torch
    import speculative_sampling_verification_02_amd as sv
    dev = gpu_util.device()
    cases = [W.config3(5, T, B=32),                                    # fused path, 16 workgroups a row
             W.gaussian_case(3, 2, 20011, "f32", T, seed=52, target_std=2.5)]  # smaller; unaligned: multipass
    for j, case in enumerate(cases):
        print(f"[noalloc] call {j}: B={case.B} gamma={case.gamma} V={case.V} {case.dtype} T={T}", flush=True)
        t = gpu_util.case_tensors(case, dev)
        ref = gpu_util.run_case(case, sv.ALGO_AUTO, tensors=t, dev=dev)
        out = _outputs(torch, case.B, case.gamma, dev)
        sv.verify_noalloc(t["target"], t["draft"], t["tokens"], t["uniforms"], case.temperature, out)
        torch.cuda.synchronize(dev)
        got = {k: v.cpu().numpy() for k, v in out.items()}
        for k in ref:
            assert np.array_equal(got[k], ref[k], equal_nan=True), (j, k)
        parity.check(case, got, where=f"noalloc call {j} T{T}")


def test_noalloc_rejects_oversized_and_bad_arguments():
    import torch
    import speculative_sampling_verification_02_amd as sv
    lib = sv.lib
    dev = gpu_util.device()
    assert sv.noalloc_limit() == 16 << 20
    fake = torch.empty(16, dtype=torch.int32, device=dev)
    p = fake.data_ptr()
    # B=4096, gamma=16, V=256000 would need far more than 16 MiB of scratch
    assert lib.spec_verify_noalloc(p, p, sv.SPEC_BF16, p, p, 4096, 16, 256000, 1.0, p, p, None, None, None,
                                   None) == sv.SPEC_ENOSPACE
    assert lib.spec_verify_noalloc(p, p, sv.SPEC_BF16, p, p, 4, 2, 100, -1.0, p, p, None, None, None,
                                   None) == sv.SPEC_EINVAL
    assert lib.spec_verify_noalloc(p, p, 7, p, p, 4, 2, 100, 1.0, p, p, None, None, None,
                                   None) == sv.SPEC_EUNSUPPORTED
    # B == 0 clears the array (a fill kernel on the stream)
    assert lib.spec_verify_noalloc(None, None, sv.SPEC_F32, None, None, 0, 2, 100, 1.0, None, None, None, None,
                                   None, None) == sv.SPEC_OK
    torch.cuda.synchronize(dev)
