"""Speculative-sampling verification on AMD Instinct MI355X (gfx950).

A thin ctypes binding over libspecverify.so, the C ABI declared in
include/specverify.h.  This module only marshals arguments: it checks tensor
dtypes, devices and contiguity, allocates outputs and workspace with torch, and
passes raw device pointers and the current HIP stream.  Every step of the
verification runs in the library's HIP kernels.  Importing fails loudly if the
library has not been built; there is no fallback path.

Build the library with `python -m speculative_sampling_verification_02_amd.build`.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EUNSUPPORTED, SPEC_ENOSPACE, SPEC_EHIP = 0, -1, -2, -3, -4
SPEC_F32, SPEC_BF16 = 0, 1
ALGO_AUTO, ALGO_MULTIPASS, ALGO_FUSED = 0, 1, 2
MAX_GAMMA = 32

_c_void_p, _c_int, _c_float, _c_size_t = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/specverify.h
SIGNATURES = {
    "spec_status_string": (ctypes.c_char_p, [_c_int]),
    "spec_verify_workspace_size": (_c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "spec_verify": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                             _c_int, _c_int, _c_int, _c_float,
                             _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                             _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_algo": (_c_int, [_c_int, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                  _c_int, _c_int, _c_int, _c_float,
                                  _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_ex": (_c_int, [_c_int, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                _c_int, _c_int, _c_int, _c_float, _c_int, _c_float, _c_float, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _c_size_t, _c_void_p]),
    "spec_filter_thresholds": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_float,
                                        _c_int, _c_float, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_filter_workspace_size": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_lmhead_logits": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "spec_stream_read": (_c_int, [_c_void_p, _c_size_t, _c_void_p, _c_int, _c_void_p]),
    "spec_lmhead_workspace_size": (_c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "spec_set_wait_limit": (None, [ctypes.c_uint]),
    "spec_verify_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                     _c_int, _c_int, _c_int, _c_float,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "spec_verify_noalloc_limit": (_c_size_t, []),
    "spec_kv_crop": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                              _c_int, _c_int, _c_int, _c_void_p]),
    "spec_kv_crop_paged": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_int, _c_int,
                                    _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_int,
                                    _c_void_p]),
    "spec_lmhead_verify": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_int, _c_int, _c_int, _c_int,
                                    _c_void_p, _c_void_p, _c_float,
                                    _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _c_size_t, _c_void_p]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m speculative_sampling_verification_02_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.spec_status_string(status).decode()} (status {status})")


def _check(status: int, where: str) -> None:
    if status != SPEC_OK:
        raise SpecVerifyError(status, where)


def status_string(status: int) -> str:
    return lib.spec_status_string(status).decode()


# ----------------------------------------------------------- torch plumbing

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _need(t, name, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(B: int, gamma: int, V: int, dtype: int = SPEC_BF16) -> int:
    return int(lib.spec_verify_workspace_size(B, gamma, V, dtype))


def verify(target_logits, draft_logits, draft_tokens, uniforms, temperature: float, *,
           algo: int = ALGO_AUTO, workspace=None, outputs=None, lenience: float = 1.0, gamma_seq=None,
           top_k: int = 0, top_p: float = 1.0):
    """One verification step on the current stream.

    target_logits [B, gamma+1, V] and draft_logits [B, gamma, V] (float32 or
    bfloat16, same dtype), draft_tokens int32 [B, gamma], uniforms float32
    [B, gamma+1]; all on the same GPU.  Returns a dict of GPU tensors:
    n_accepted int32 [B], next_token int32 [B], alpha / p_draft / q_draft
    float32 [B, gamma].  `outputs` may supply that dict preallocated.

    `workspace` is a uint8 GPU tensor of at least workspace_size() bytes that
    is all-zero before its first use; every completed call leaves it zero, so
    one tensor serves a whole serving loop.  Without one, a zeroed tensor is
    allocated for this call.  n_accepted = -1 marks a sequence whose result
    was lost because a wait gave up (the device was shared, see
    include/specverify.h); the workspace must then be zeroed again
    (workspace.zero_()) before its next use.

    top_k / top_p (filters of both models' rows), lenience (l in (0, 1]) and
    gamma_seq (int32 [B] on the same GPU, each gamma_b in [0, gamma]) are the
    extensions of spec_verify_ex: the adjusted distributions, q scaled by l in
    the accept test and the residual, and per-sequence draft counts in the
    padded layout (positions past gamma_b report NaN).
    """
    torch = _torch()
    dev = target_logits.device
    _need(target_logits, "target_logits")
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    if tuple(draft_logits.shape) != (B, gamma, V):
        raise ValueError(f"draft_logits must be [{B}, {gamma}, {V}], got {tuple(draft_logits.shape)}")
    if draft_logits.dtype != target_logits.dtype:
        raise TypeError("target_logits and draft_logits must share a dtype")
    if tuple(draft_tokens.shape) != (B, gamma) or tuple(uniforms.shape) != (B, g1):
        raise ValueError("draft_tokens must be [B, gamma] and uniforms [B, gamma+1]")
    _need(draft_logits, "draft_logits", device=dev)
    _need(draft_tokens, "draft_tokens", torch.int32, dev)
    _need(uniforms, "uniforms", torch.float32, dev)
    if gamma_seq is not None:
        _need(gamma_seq, "gamma_seq", torch.int32, dev)
        if tuple(gamma_seq.shape) != (B,):
            raise ValueError(f"gamma_seq must be [{B}]")
    dt = _dtype_code(target_logits)
    if outputs is None:
        outputs = {
            "n_accepted": torch.empty(B, dtype=torch.int32, device=dev),
            "next_token": torch.empty(B, dtype=torch.int32, device=dev),
            "alpha": torch.empty(B, gamma, dtype=torch.float32, device=dev),
            "p_draft": torch.empty(B, gamma, dtype=torch.float32, device=dev),
            "q_draft": torch.empty(B, gamma, dtype=torch.float32, device=dev),
        }
    need = workspace_size(B, gamma, V, dt)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.spec_verify_ex(*_verify_args(algo, target_logits, draft_logits, dt, draft_tokens, uniforms,
                                            B, gamma, V, temperature, top_k, top_p, lenience, gamma_seq,
                                            outputs, workspace, dev)),
           "spec_verify")
    return outputs


def verify_noalloc(target_logits, draft_logits, draft_tokens, uniforms, temperature: float, outputs: dict):
    """spec_verify_noalloc: verify() with the library's own per-device scratch
    instead of a workspace, for callers that cannot allocate.  `outputs` is
    the dict of preallocated output tensors (n_accepted, next_token, alpha,
    p_draft, q_draft, as verify() returns them); nothing is allocated here."""
    torch = _torch()
    dev = target_logits.device
    _need(target_logits, "target_logits")
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    if tuple(draft_logits.shape) != (B, gamma, V) or draft_logits.dtype != target_logits.dtype:
        raise ValueError(f"draft_logits must be [{B}, {gamma}, {V}] with the target's dtype")
    if tuple(draft_tokens.shape) != (B, gamma) or tuple(uniforms.shape) != (B, g1):
        raise ValueError("draft_tokens must be [B, gamma] and uniforms [B, gamma+1]")
    _need(draft_logits, "draft_logits", device=dev)
    _need(draft_tokens, "draft_tokens", torch.int32, dev)
    _need(uniforms, "uniforms", torch.float32, dev)
    for name, shape in (("n_accepted", (B,)), ("next_token", (B,))):
        _need(outputs[name], name, torch.int32, dev)
        if tuple(outputs[name].shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    for name in ("alpha", "p_draft", "q_draft"):
        if outputs.get(name) is not None:
            _need(outputs[name], name, torch.float32, dev)
            if tuple(outputs[name].shape) != (B, gamma):
                raise ValueError(f"{name} must be {(B, gamma)}")
    _check(lib.spec_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits),
                                   _ptr(draft_tokens), _ptr(uniforms), B, gamma, V, float(temperature),
                                   _ptr(outputs["n_accepted"]), _ptr(outputs["next_token"]),
                                   _ptr(outputs.get("alpha")), _ptr(outputs.get("p_draft")),
                                   _ptr(outputs.get("q_draft")), _stream(dev)), "spec_verify_noalloc")
    return outputs


def _cache_array(caches):
    """A host array of the caches' device pointers (kept alive by the caller)."""
    if not caches:
        return None, 0
    ptrs = (ctypes.c_void_p * len(caches))(*[c.data_ptr() for c in caches])
    return ptrs, len(caches)


def kv_crop(caches, seq_len, n_accepted, appended: int, keep_extra: int = 0, clear: bool = True):
    """spec_kv_crop on the current stream.  caches: contiguous GPU tensors
    [B, H, S_max, D] (any element type; entries of D elements, a multiple of
    16 bytes); seq_len: int32 [B] (updated in place on the device); n_accepted:
    int32 [B] as verify() returned it."""
    torch = _torch()
    dev = seq_len.device
    _need(seq_len, "seq_len", torch.int32)
    _need(n_accepted, "n_accepted", torch.int32, dev)
    B = seq_len.numel()
    H = S_max = entry = 1
    for c in caches:
        _need(c, "cache", device=dev)
        if c.dim() != 4 or c.shape[0] != B:
            raise ValueError("every cache must be [B, H, S_max, D]")
    if caches:
        _, H, S_max, D = caches[0].shape
        entry = D * caches[0].element_size()
        if any(tuple(c.shape) != tuple(caches[0].shape) or c.element_size() != caches[0].element_size()
               for c in caches):
            raise ValueError("the caches must share shape and element size")
    ptrs, n = _cache_array(list(caches))
    _check(lib.spec_kv_crop(ptrs, n, B, H, S_max, max(entry, 16), _ptr(seq_len), _ptr(n_accepted), int(appended),
                            int(keep_extra), int(bool(clear)), _stream(dev)), "spec_kv_crop")


def kv_crop_paged(caches, block_table, seq_len, n_accepted, appended: int, free_pages, free_count,
                  keep_extra: int = 0, clear: bool = True, page_size: int = 0, num_pages: int = 0,
                  token_bytes: int = 16):
    """spec_kv_crop_paged on the current stream.  caches: GPU tensors
    [num_pages, page_size, ...] (the rest of a page slot is one token's
    entries, a multiple of 16 bytes); block_table int32 [B, max_blocks];
    seq_len int32 [B]; free_pages int32 [>= num_pages]; free_count int32 [1]
    (all updated in place on the device).  page_size / num_pages /
    token_bytes come from the caches when they are given."""
    torch = _torch()
    dev = seq_len.device
    for name, t in (("block_table", block_table), ("seq_len", seq_len), ("n_accepted", n_accepted),
                    ("free_pages", free_pages), ("free_count", free_count)):
        _need(t, name, torch.int32, dev)
    B, max_blocks = block_table.shape
    if caches:
        num_pages, page_size = caches[0].shape[0], caches[0].shape[1]
        token_bytes = caches[0][0, 0].numel() * caches[0].element_size()
        for c in caches:
            _need(c, "cache", device=dev)
            if tuple(c.shape) != tuple(caches[0].shape) or c.element_size() != caches[0].element_size():
                raise ValueError("the caches must share shape and element size")
    ptrs, n = _cache_array(list(caches))
    _check(lib.spec_kv_crop_paged(ptrs, n, int(num_pages), int(page_size), int(token_bytes), _ptr(block_table), B,
                                  max_blocks, _ptr(seq_len), _ptr(n_accepted), int(appended), int(keep_extra),
                                  int(bool(clear)), _ptr(free_pages), _ptr(free_count), free_pages.numel(),
                                  _stream(dev)), "spec_kv_crop_paged")


def noalloc_limit() -> int:
    """Bytes of the per-device array spec_verify_noalloc uses."""
    return int(lib.spec_verify_noalloc_limit())


def set_wait_limit(polls: int) -> None:
    """Polls after which every cross-workgroup wait of later launches gives up
    (spec_set_wait_limit); 0 restores the default."""
    lib.spec_set_wait_limit(int(polls))


def filter_workspace_size(B: int, gamma: int, V: int) -> int:
    """Bytes of the optional filter_thresholds workspace (spec_filter_workspace_size)."""
    return int(lib.spec_filter_workspace_size(int(B), int(gamma), int(V)))


def filter_thresholds(target_logits, draft_logits, temperature: float, top_k: int = 0, top_p: float = 1.0,
                      workspace=None):
    """Per-row keep thresholds of top-k / top-p (spec_filter_thresholds).

    target_logits [B, gamma+1, V] and draft_logits [B, gamma, V] (float32 or
    bfloat16) on one GPU; temperature > 0.  workspace: None, or a zeroed uint8
    GPU tensor of at least filter_workspace_size(B, gamma, V) bytes (left
    zeroed), which lets a top-k of at most 64 select from chunk candidate lists.
    Returns float32 GPU tensors (target [B, gamma+1], draft [B, gamma]): a row
    keeps the tokens whose logit is >= its threshold (-inf: the whole row)."""
    torch = _torch()
    dev = target_logits.device
    _need(target_logits, "target_logits")
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    if tuple(draft_logits.shape) != (B, gamma, V) or draft_logits.dtype != target_logits.dtype:
        raise ValueError("draft_logits must be [B, gamma, V] with the target's dtype")
    _need(draft_logits, "draft_logits", device=dev)
    thr = torch.empty(B * g1 + B * gamma, dtype=torch.float32, device=dev)
    ws, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
        ws, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib.spec_filter_thresholds(_ptr(target_logits), _ptr(draft_logits) if gamma else None,
                                      _dtype_code(target_logits), B, gamma, V, float(temperature), int(top_k),
                                      float(top_p), _ptr(thr), ws, ws_bytes, _stream(dev)), "spec_filter_thresholds")
    return thr[:B * g1].view(B, g1), thr[B * g1:].view(B, gamma)


def stream_read(buffer, sink, blocks: int):
    """One plain streaming read of `buffer` (a 16-byte aligned GPU tensor) on
    the current stream; `sink` is a GPU int32 tensor of at least `blocks`."""
    _need(buffer, "buffer")
    _need(sink, "sink", device=buffer.device)
    if sink.numel() * sink.element_size() < 4 * int(blocks):
        raise ValueError("sink must hold one 32-bit word per workgroup")
    nbytes = buffer.numel() * buffer.element_size()
    _check(lib.spec_stream_read(_ptr(buffer), nbytes, _ptr(sink), int(blocks), _stream(buffer.device)),
           "spec_stream_read")


def _verify_args(algo, target_logits, draft_logits, dt, draft_tokens, uniforms, B, gamma, V, temperature,
                 top_k, top_p, lenience, gamma_seq, outputs, workspace, dev):
    return (algo, _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens), _ptr(uniforms),
            B, gamma, V, float(temperature), int(top_k), float(top_p), float(lenience), _ptr(gamma_seq),
            _ptr(outputs["n_accepted"]), _ptr(outputs["next_token"]), _ptr(outputs.get("alpha")),
            _ptr(outputs.get("p_draft")), _ptr(outputs.get("q_draft")),
            _ptr(workspace), workspace.numel(), _stream(dev))


def prepare_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature: float, *,
                   algo: int = ALGO_AUTO, workspace, outputs, lenience: float = 1.0, gamma_seq=None,
                   top_k: int = 0, top_p: float = 1.0):
    """Checks the arguments of verify() once and returns a callable that
    launches that same verification again (same tensors, current stream at
    preparation) with no per-call Python work beyond the C call, for loops
    whose host time per step must stay well under the kernel's.  The callable
    holds references to every tensor it launches on, so they stay allocated
    while it lives; their shapes and contents are the caller's to keep."""
    verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, algo=algo, workspace=workspace,
           outputs=outputs, lenience=lenience, gamma_seq=gamma_seq, top_k=top_k, top_p=top_p)
    B, g1, V = target_logits.shape
    args = _verify_args(algo, target_logits, draft_logits, _dtype_code(target_logits), draft_tokens, uniforms,
                        B, g1 - 1, V, temperature, top_k, top_p, lenience, gamma_seq, outputs, workspace,
                        target_logits.device)
    fn = lib.spec_verify_ex
    keep = (target_logits, draft_logits, draft_tokens, uniforms, gamma_seq, workspace, dict(outputs))

    def launch():
        status = fn(*args)
        if status != 0:
            _check(status, "spec_verify")

    launch.tensors = keep  # the device buffers behind the raw pointers in args
    return launch


def lmhead_workspace_size(B: int, gamma: int, d: int, V: int) -> int:
    """Bytes of device workspace spec_lmhead_verify needs (zero on entry)."""
    return int(lib.spec_lmhead_workspace_size(B, gamma, d, V))


def lmhead_logits(hidden, W, out=None):
    """logits[M, V] = hidden[M, d] @ W[d, V] (bf16 in, fp32 accumulate and out)."""
    torch = _torch()
    dev = hidden.device
    _need(hidden, "hidden", torch.bfloat16)
    _need(W, "W", torch.bfloat16, dev)
    M, d = hidden.shape
    V = W.shape[1]
    if W.shape[0] != d:
        raise ValueError("W must be [d, V]")
    if out is None:
        out = torch.empty(M, V, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    _check(lib.spec_lmhead_logits(_ptr(hidden), _ptr(W), M, d, V, _ptr(out), _stream(dev)),
           "spec_lmhead_logits")
    return out


def lmhead_verify(hidden, W_target, W_draft, B: int, gamma: int, draft_tokens, uniforms,
                  temperature: float, hidden_draft=None, workspace=None, outputs=None):
    """LM heads of both models over the verified positions, then the verification.

    hidden bf16 [B*(gamma+1), d]; W_target / W_draft bf16 [d, V]; hidden_draft
    bf16 [B*gamma, d] or None (rows 0..gamma-1 of each sequence in `hidden`).
    Returns the verify outputs plus the fp32 target_logits and draft_logits
    (in `outputs` when given: a dict of tensors of those names and shapes).
    """
    torch = _torch()
    dev = hidden.device
    _need(hidden, "hidden", torch.bfloat16)
    _need(W_target, "W_target", torch.bfloat16, dev)
    _need(W_draft, "W_draft", torch.bfloat16, dev)
    if hidden_draft is not None:
        _need(hidden_draft, "hidden_draft", torch.bfloat16, dev)
    _need(draft_tokens, "draft_tokens", torch.int32, dev)
    _need(uniforms, "uniforms", torch.float32, dev)
    d, V = W_target.shape
    if tuple(hidden.shape) != (B * (gamma + 1), d):
        raise ValueError("hidden must be [B*(gamma+1), d]")
    out = outputs if outputs is not None else {
        "target_logits": torch.empty(B, gamma + 1, V, dtype=torch.float32, device=dev),
        "draft_logits": torch.empty(B, gamma, V, dtype=torch.float32, device=dev),
        "n_accepted": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "alpha": torch.empty(B, gamma, dtype=torch.float32, device=dev),
        "p_draft": torch.empty(B, gamma, dtype=torch.float32, device=dev),
        "q_draft": torch.empty(B, gamma, dtype=torch.float32, device=dev),
    }
    if outputs is not None:
        for name, shape, dt in (("target_logits", (B, gamma + 1, V), torch.float32),
                                ("draft_logits", (B, gamma, V), torch.float32),
                                ("n_accepted", (B,), torch.int32), ("next_token", (B,), torch.int32),
                                ("alpha", (B, gamma), torch.float32), ("p_draft", (B, gamma), torch.float32),
                                ("q_draft", (B, gamma), torch.float32)):
            _need(out[name], name, dt, dev)
            if tuple(out[name].shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
    need = int(lib.spec_lmhead_workspace_size(B, gamma, d, V))
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.spec_lmhead_verify(
        _ptr(hidden), _ptr(hidden_draft), _ptr(W_target), _ptr(W_draft), B, gamma, d, V,
        _ptr(draft_tokens), _ptr(uniforms), float(temperature),
        _ptr(out["target_logits"]), _ptr(out["draft_logits"]),
        _ptr(out["n_accepted"]), _ptr(out["next_token"]), _ptr(out["alpha"]),
        _ptr(out["p_draft"]), _ptr(out["q_draft"]),
        _ptr(workspace), workspace.numel(), _stream(dev)), "spec_lmhead_verify")
    return out
