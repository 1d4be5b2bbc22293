"""Python binding of the gfx950 O(N)-memory attention library (libfa.so).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory (output and workspace tensors) and the current
HIP stream.  The functions carry the C entry points' names:

    o, lse = fa_fwd(q, k, v, seg=None, scale=None, causal=True)
    dq, dk, dv = fa_bwd(q, k, v, o, do, lse, seg=None, scale=None, causal=True)
    nll, lse, tlogit = fa_lce_fwd(h, w, targets)
    dh, dw = fa_lce_bwd(h, w, targets, lse, dnll)

q, o, do are contiguous (B, H, N, D) CUDA tensors and k, v (B, Hkv, N, D)
with Hkv dividing H (torch.bfloat16 or torch.float32, D in {64, 96, 128}); seg
is None or a contiguous (B, N) int32 CUDA tensor of non-decreasing segment
ids; lse is (B, H, N) float32.  The fused linear cross-entropy takes bf16
hidden states h (N, D) and head w (V, D) and int32 targets (N,).  A refused
call raises FaError naming the reason; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FaError", "fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_workspace_bytes", "fa_check_seg",
           "fa_status_string", "flash_attention", "fa_lce_fwd", "fa_lce_bwd", "fa_lce_workspace_bytes",
           "linear_cross_entropy", "library_path", "load_library", "FA_BF16", "FA_FP32"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa.so")
FA_BF16, FA_FP32 = 0, 1
FA_ERR_SEG = 8
FA_ERR_SCRATCH = 11
FA_NOALLOC_MAX_BYTES = 32 << 20
_lib = None


class FaError(RuntimeError):
    """A refused or failed library call; ``status`` is the fa_status code."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (fa_status {status})")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfa.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m memory_efficient_attention_amd.build`")
    # torch first: its bundled HIP runtime (SONAME libamdhip64.so.7) must be the
    # one in the process, so that libfa.so binds to it and streams/pointers
    # from torch are valid in the library.  Loaded the other way round, torch
    # would map a second runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_workspace_bytes.restype = sz
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, f, i, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, f, i, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, f, i, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp,
                                 vp]
    lib.fa_bwd_timed.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, f, i, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_lce_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_lce_workspace_bytes.restype = sz
    lib.fa_lce_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.fa_lce_fwd.restype = i
    lib.fa_lce_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.fa_lce_bwd.restype = i
    lib.fa_check_seg.argtypes = [vp, i, i]
    lib.fa_check_seg.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_workspace_bytes(B: int, H: int, N: int, D: int, has_seg: bool, for_bwd: bool) -> int:
    return int(load_library().fa_workspace_bytes(B, H, N, D, int(bool(has_seg)), int(bool(for_bwd))))


def fa_check_seg(seg) -> None:
    """Validate a host (CPU) copy of seg; raises FaError if ids decrease in a row."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(seg.cpu() if hasattr(seg, "cpu") else seg, dtype=np.int32))
    if a.ndim != 2:
        raise ValueError("seg must be (B, N)")
    st = load_library().fa_check_seg(a.ctypes.data, a.shape[0], a.shape[1])
    if st:
        raise FaError(st, "fa_check_seg")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    return 99   # the library refuses it with FA_ERR_DTYPE


def _check_tensor(name, t, shape, dtype, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _seg_ptr(seg, B, N, device):
    import torch
    if seg is None:
        return None
    _check_tensor("seg", seg, (B, N), torch.int32, device)
    return seg.data_ptr()


def _stream():
    """The current stream of the current device (calls run under the device
    of their tensors, see _on)."""
    import torch
    return torch.cuda.current_stream().cuda_stream


def _on(device):
    """Make the tensors' device current for the library call, so that the
    kernels and the stream are that device's."""
    import torch
    return torch.cuda.device(device)


def _workspace(ws, nbytes, device, min_bytes=0):
    """The caller's workspace, checked (device, layout, size: a caller that
    passes one gets no allocation), or a new one of max(nbytes, min_bytes)
    bytes (None when the call needs none).  Returns (tensor or None, its size
    in bytes)."""
    import torch
    if ws is None:
        if nbytes == 0 and min_bytes == 0:
            return None, 0
        ws = torch.empty(max(nbytes, min_bytes), dtype=torch.uint8, device=device)
        return ws, ws.numel()
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    size = ws.numel() * ws.element_size()
    if size < nbytes:
        raise ValueError(f"workspace has {size} bytes, {nbytes} needed")
    return ws, size


def _kv_heads(q, k) -> int:
    """Key/value heads of k (grouped-query attention when fewer than q's)."""
    if k.dim() != 4:
        raise ValueError("k must be (B, Hkv, N, D)")
    return int(k.shape[1])


def _segment_flag(ws, seg, check_seg, where):
    """With check_seg, read the device's segment-order flag (workspace word 0,
    set by the schedule when ids decrease along a row) and raise FaError
    (FA_ERR_SEG) if it is set.  This waits for the call to finish."""
    if not check_seg or seg is None:
        return
    import torch
    if int(ws[:4].view(torch.int32).item()) != 0:
        raise FaError(FA_ERR_SEG, where)


def fa_fwd(q, k, v, seg=None, scale=None, causal=True, out=None, lse=None, workspace=None,
           check_seg=False):
    """Forward pass; returns (o, lse).  q is (B, H, N, D); k and v are
    (B, Hkv, N, D) with Hkv dividing H (query head h reads key/value head
    h // (H // Hkv)).  check_seg: after the call, wait for it and raise
    FaError if the device found segment ids that decrease along a row (their
    outputs are then unspecified)."""
    import torch
    B, H, N, D = q.shape
    Hkv = _kv_heads(q, k)
    dev = q.device
    _check_tensor("q", q, (B, H, N, D), q.dtype)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, Hkv, N, D), q.dtype, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor("o", o, (B, H, N, D), q.dtype, dev)
    _check_tensor("lse", lse_t, (B, H, N), torch.float32, dev)
    seg_p = _seg_ptr(seg, B, N, dev)
    lib = load_library()
    nbytes = lib.fa_workspace_bytes(B, H, N, D, int(seg is not None), 0)
    ws, ws_bytes = _workspace(workspace, nbytes, dev)
    with _on(dev):
        st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), seg_p, ctypes.c_float(scale),
                        int(bool(causal)), o.data_ptr(), lse_t.data_ptr(), B, H, Hkv, N, D,
                        _dtype_code(q), ws.data_ptr() if ws is not None else None, ws_bytes, _stream())
    if st:
        raise FaError(st, "fa_fwd")
    _segment_flag(ws, seg, check_seg, "fa_fwd")
    return o, lse_t


def fa_bwd(q, k, v, o, do, lse, seg=None, scale=None, causal=True, dq=None, dk=None, dv=None,
           workspace=None, events=None, check_seg=False):
    """Backward pass from dO; returns (dq, dk, dv).  check_seg as in fa_fwd.

    ``events``: optional sequence of 3 raw hipEvent_t handles (ints or None)
    recorded before dQ, between dQ and dK/dV, and after dK/dV
    (fa_bwd_timed in the C ABI)."""
    import torch
    B, H, N, D = q.shape
    Hkv = _kv_heads(q, k)
    dev = q.device
    for name, t in (("q", q), ("o", o), ("do", do)):
        _check_tensor(name, t, (B, H, N, D), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, Hkv, N, D), q.dtype, dev)
    _check_tensor("lse", lse, (B, H, N), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, (B, H, N, D), q.dtype, dev)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_tensor(name, t, (B, Hkv, N, D), q.dtype, dev)
    seg_p = _seg_ptr(seg, B, N, dev)
    lib = load_library()
    nbytes = lib.fa_workspace_bytes(B, H, N, D, int(seg is not None), 1)
    ws, ws_bytes = _workspace(workspace, nbytes, dev)
    with _on(dev):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                lse.data_ptr(), seg_p, ctypes.c_float(scale), int(bool(causal)),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, D, _dtype_code(q),
                ws.data_ptr(), ws_bytes, _stream())
        if events is None:
            st = lib.fa_bwd(*args)
        else:
            if len(events) != 3:
                raise ValueError("events: 3 hipEvent_t handles (or None)")
            ev = (ctypes.c_void_p * 3)(*[e or None for e in events])
            st = lib.fa_bwd_timed(*args, ev)
    if st:
        raise FaError(st, "fa_bwd")
    _segment_flag(ws, seg, check_seg, "fa_bwd")
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, do, lse, seg=None, scale=None, causal=True, dq=None, dk=None, dv=None):
    """fa_bwd without a workspace: the library uses its own static device
    array (FA_NOALLOC_MAX_BYTES per GPU), so the call allocates nothing when
    dq, dk and dv are given.  Calls that overlap on one GPU race on that
    array.  Shapes needing more workspace raise FaError (FA_ERR_SCRATCH)."""
    import torch
    B, H, N, D = q.shape
    Hkv = _kv_heads(q, k)
    dev = q.device
    for name, t in (("q", q), ("o", o), ("do", do)):
        _check_tensor(name, t, (B, H, N, D), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, Hkv, N, D), q.dtype, dev)
    _check_tensor("lse", lse, (B, H, N), torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, (B, H, N, D), q.dtype, dev)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_tensor(name, t, (B, Hkv, N, D), q.dtype, dev)
    seg_p = _seg_ptr(seg, B, N, dev)
    lib = load_library()
    with _on(dev):
        st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), seg_p, ctypes.c_float(scale), int(bool(causal)),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, D,
                                _dtype_code(q), _stream())
    if st:
        raise FaError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def flash_attention(q, k, v, scale=None, causal=True, segments=None):
    """Differentiable attention through fa_fwd / fa_bwd (torch.autograd.Function)."""
    import torch

    class _Fn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q_, k_, v_):
            o, lse = fa_fwd(q_, k_, v_, segments, scale, causal)
            ctx.save_for_backward(q_, k_, v_, o, lse)
            return o

        @staticmethod
        def backward(ctx, do):
            q_, k_, v_, o, lse = ctx.saved_tensors
            return fa_bwd(q_, k_, v_, o, do.contiguous(), lse, segments, scale, causal)

    return _Fn.apply(q, k, v)


# ---------------------------------------------------------------- linear cross-entropy

def fa_lce_workspace_bytes(N: int, V: int, D: int, for_bwd: bool) -> int:
    return int(load_library().fa_lce_workspace_bytes(N, V, D, int(bool(for_bwd))))


def fa_lce_fwd(h, w, targets, workspace=None):
    """Fused linear cross-entropy forward; returns (nll, lse, tlogit), each (N,)
    fp32.  h (N, D) and w (V, D) bf16, targets (N,) int32."""
    import torch
    N, D = h.shape
    V = w.shape[0]
    dev = h.device
    _check_tensor("h", h, (N, D), h.dtype)
    _check_tensor("w", w, (V, D), h.dtype, dev)
    _check_tensor("targets", targets, (N,), torch.int32, dev)
    nll, lse, tz = (torch.empty(N, dtype=torch.float32, device=dev) for _ in range(3))
    lib = load_library()
    nbytes = lib.fa_lce_workspace_bytes(N, V, D, 0)
    ws, ws_bytes = _workspace(workspace, nbytes, dev, 256)
    with _on(dev):
        st = lib.fa_lce_fwd(h.data_ptr(), w.data_ptr(), targets.data_ptr(), nll.data_ptr(), lse.data_ptr(),
                            tz.data_ptr(), N, V, D, _dtype_code(h), ws.data_ptr(), ws_bytes, _stream())
    if st:
        raise FaError(st, "fa_lce_fwd")
    return nll, lse, tz


def fa_lce_bwd(h, w, targets, lse, dnll, need_dw=True, workspace=None):
    """Backward from per-token NLL gradients dnll (N,) fp32; returns (dh, dw)
    (dw is None when need_dw is False)."""
    import torch
    N, D = h.shape
    V = w.shape[0]
    dev = h.device
    _check_tensor("h", h, (N, D), h.dtype)
    _check_tensor("w", w, (V, D), h.dtype, dev)
    _check_tensor("targets", targets, (N,), torch.int32, dev)
    _check_tensor("lse", lse, (N,), torch.float32, dev)
    _check_tensor("dnll", dnll, (N,), torch.float32, dev)
    dh = torch.empty_like(h)
    dw = torch.empty_like(w) if need_dw else None
    lib = load_library()
    nbytes = lib.fa_lce_workspace_bytes(N, V, D, 1)
    ws, ws_bytes = _workspace(workspace, nbytes, dev, 256)
    with _on(dev):
        st = lib.fa_lce_bwd(h.data_ptr(), w.data_ptr(), targets.data_ptr(), lse.data_ptr(), dnll.data_ptr(),
                            dh.data_ptr(), dw.data_ptr() if dw is not None else None, N, V, D, _dtype_code(h),
                            ws.data_ptr(), ws_bytes, _stream())
    if st:
        raise FaError(st, "fa_lce_bwd")
    return dh, dw


def linear_cross_entropy(h, w, targets):
    """Differentiable per-token loss through fa_lce_fwd / fa_lce_bwd: the NLL
    of softmax(h w^T) at `targets`, an (N,) fp32 tensor.  Reducing it (mean,
    sum) is the caller's step; its gradient reaches fa_lce_bwd per token."""
    import torch

    class _Fn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, h_, w_):
            nll, lse, _ = fa_lce_fwd(h_, w_, targets)
            ctx.save_for_backward(h_, w_, lse)
            return nll

        @staticmethod
        def backward(ctx, g):
            h_, w_, lse = ctx.saved_tensors
            dh, dw = fa_lce_bwd(h_, w_, targets, lse, g.contiguous(), need_dw=ctx.needs_input_grad[1])
            return dh, dw

    return _Fn.apply(h, w)
