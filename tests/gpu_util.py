"""Moving seeded numpy cases onto the GPU and running the library on them (test helper)."""

from __future__ import annotations

import numpy as np


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def to_gpu(arr: np.ndarray, dtype: str, dev):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def case_tensors(case, dev):
    import torch
    return dict(
        target=to_gpu(case.target, case.dtype, dev),
        draft=to_gpu(case.draft, case.dtype, dev),
        tokens=torch.from_numpy(np.ascontiguousarray(case.tokens, dtype=np.int32)).to(dev),
        uniforms=torch.from_numpy(np.ascontiguousarray(case.uniforms, dtype=np.float32)).to(dev),
    )


def run_case(case, algo, tensors=None, dev=None, lenience: float = 1.0, gamma_seq=None, workspace=None,
             top_k: int = 0, top_p: float = 1.0):
    """gamma_seq: numpy int [B] (per-sequence draft counts) or None."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    dev = dev or device()
    t = tensors or case_tensors(case, dev)
    gs = None if gamma_seq is None else torch.from_numpy(np.ascontiguousarray(gamma_seq, dtype=np.int32)).to(dev)
    try:
        out = sv.verify(t["target"], t["draft"], t["tokens"], t["uniforms"], case.temperature, algo=algo,
                        lenience=lenience, gamma_seq=gs, workspace=workspace, top_k=top_k, top_p=top_p)
    except sv.SpecVerifyError as e:
        if e.status == sv.SPEC_EUNSUPPORTED and algo == sv.ALGO_FUSED:
            import pytest
            pytest.skip("the fused path declines this shape (unaligned rows or too long a row)")
        raise
    torch.cuda.synchronize(dev)
    return {k: v.cpu().numpy() for k, v in out.items()}


def gpu_thresholds(case, top_k: int, top_p: float, dev=None, tensors=None):
    """The GPU's keep thresholds for a case ([B, 2 gamma + 1]: target rows, then
    draft rows), from spec_filter_thresholds with a workspace -- the kernels
    the verification itself launches first (its workspace holds the filter's:
    with top-p alone the streaming nucleus launches, whose thresholds may
    differ from the row kernel's by a tie group in rows within the nucleus
    band)."""
    import torch
    import speculative_sampling_verification_02_amd as sv
    dev = dev or device()
    t = tensors or case_tensors(case, dev)
    ws = torch.zeros(sv.filter_workspace_size(case.B, case.gamma, case.V), dtype=torch.uint8, device=dev)
    gt, gd = sv.filter_thresholds(t["target"], t["draft"], case.temperature, top_k, top_p, workspace=ws)
    return np.concatenate([gt.cpu().numpy(), gd.cpu().numpy()], axis=1)
