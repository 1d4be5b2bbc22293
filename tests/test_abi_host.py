"""The C ABI on the host: the library loads, exports what include/fa.h declares,
and refuses bad arguments with the right status before any HIP call.

No compute runs here (this suite also runs on machines without a GPU); the
tensor pointers passed are fake, non-null integers that a refusal never touches.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_DTYPE = 0, 1, 2, 3, 4
FA_ERR_WORKSPACE, FA_ERR_ALIGN, FA_ERR_SCALE, FA_ERR_SEG, FA_ERR_HIP, FA_ERR_DEVICE = 5, 6, 7, 8, 9, 10
FA_ERR_SCRATCH = 11


@pytest.fixture(scope="module")
def lib():
    import memory_efficient_attention_amd as fa
    if not os.path.exists(fa.library_path()):
        fa_build = pytest.importorskip("memory_efficient_attention_amd.build")
        fa_build.build()
    return fa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_status_values_match():
    text = open(HEADER).read()
    vals = dict((n, int(v)) for n, v in re.findall(r"\b(FA_\w+)\s*=\s*(\d+)", text))
    assert vals["FA_OK"] == FA_OK and vals["FA_ERR_DEVICE"] == FA_ERR_DEVICE
    assert vals["FA_ERR_ALIGN"] == FA_ERR_ALIGN and vals["FA_ERR_SEG"] == FA_ERR_SEG
    assert vals["FA_ERR_SCRATCH"] == FA_ERR_SCRATCH


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == ["fa_bwd", "fa_bwd_noalloc", "fa_bwd_timed", "fa_check_seg", "fa_fwd", "fa_lce_bwd",
                        "fa_lce_fwd", "fa_lce_workspace_bytes", "fa_status_string", "fa_workspace_bytes"]
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (fa_\w+)", out)))
    assert exported == declared          # and nothing else leaks out of the library
    for name in declared:
        assert hasattr(lib, name)


def test_no_undefined_library_symbols(lib):
    """Every kernel stub and helper of the library is defined in it (a missing
    host stub only shows up as an undefined symbol when the GPU loader binds)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", lib._name], capture_output=True,
                         text=True).stdout
    own = [l for l in out.splitlines() if "_ZN2fa" in l]
    assert not own, own


GOOD = dict(B=1, H=2, N=64, D=64, dtype=0, scale=0.125)
P = 0x100000   # fake, 256-aligned, never dereferenced


def _fwd(lib, q=P, k=P, v=P, seg=None, scale=0.125, causal=1, o=P, lse=P, B=1, H=2, Hkv=None,
         N=64, D=64, dtype=0, ws=None, ws_bytes=0):
    Hkv = H if Hkv is None else Hkv
    return lib.fa_fwd(q, k, v, seg, ctypes.c_float(scale), causal, o, lse, B, H, Hkv, N, D, dtype, ws,
                      ws_bytes, None)


def _bwd(lib, q=P, k=P, v=P, o=P, do=P, lse=P, seg=None, scale=0.125, causal=1, dq=P, dk=P, dv=P,
         B=1, H=2, Hkv=None, N=64, D=64, dtype=0, ws=P, ws_bytes=1 << 30):
    Hkv = H if Hkv is None else Hkv
    return lib.fa_bwd(q, k, v, o, do, lse, seg, ctypes.c_float(scale), causal, dq, dk, dv, B, H, Hkv, N,
                      D, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), FA_ERR_NULL), (dict(lse=None), FA_ERR_NULL), (dict(o=None), FA_ERR_NULL),
    (dict(B=0), FA_ERR_SHAPE), (dict(H=-1), FA_ERR_SHAPE), (dict(N=0), FA_ERR_SHAPE),
    (dict(Hkv=0), FA_ERR_SHAPE), (dict(Hkv=-2), FA_ERR_SHAPE), (dict(H=6, Hkv=4), FA_ERR_SHAPE),
    (dict(H=2, Hkv=4), FA_ERR_SHAPE),
    (dict(N=(1 << 22) + 1), FA_ERR_SHAPE), (dict(N=1 << 22, D=128, dtype=1), FA_ERR_SHAPE), (dict(B=1 << 16, H=1 << 10, N=1 << 10), FA_ERR_SHAPE),
    (dict(D=80), FA_ERR_HEAD_DIM), (dict(D=32), FA_ERR_HEAD_DIM), (dict(D=256), FA_ERR_HEAD_DIM),
    (dict(D=112), FA_ERR_HEAD_DIM), (dict(D=0), FA_ERR_HEAD_DIM),
    (dict(dtype=2), FA_ERR_DTYPE), (dict(dtype=-1), FA_ERR_DTYPE),
    (dict(scale=float("nan")), FA_ERR_SCALE), (dict(scale=float("inf")), FA_ERR_SCALE),
    (dict(scale=0.0), FA_ERR_SCALE), (dict(scale=-1.0), FA_ERR_SCALE),
    (dict(q=P + 8), FA_ERR_ALIGN), (dict(v=P + 2), FA_ERR_ALIGN), (dict(lse=P + 2), FA_ERR_ALIGN),
    (dict(seg=P + 1, ws=P, ws_bytes=1 << 20), FA_ERR_ALIGN),
    (dict(seg=P), FA_ERR_WORKSPACE), (dict(seg=P, ws=P, ws_bytes=16), FA_ERR_WORKSPACE),
    (dict(seg=P, ws=P + 16, ws_bytes=1 << 20), FA_ERR_ALIGN),
])
def test_fwd_refusals(lib, kw, status):
    assert _fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(do=None), FA_ERR_NULL), (dict(dv=None), FA_ERR_NULL), (dict(lse=None), FA_ERR_NULL),
    (dict(N=-5), FA_ERR_SHAPE), (dict(H=8, Hkv=3), FA_ERR_SHAPE), (dict(D=80), FA_ERR_HEAD_DIM),
    (dict(dtype=7), FA_ERR_DTYPE),
    (dict(scale=float("-inf")), FA_ERR_SCALE), (dict(dk=P + 4), FA_ERR_ALIGN),
    (dict(ws=None), FA_ERR_WORKSPACE), (dict(ws_bytes=100), FA_ERR_WORKSPACE),
    (dict(ws=P + 64), FA_ERR_ALIGN),
])
def test_bwd_refusals(lib, kw, status):
    assert _bwd(lib, **kw) == status


def _bwd_noalloc(lib, q=P, k=P, v=P, o=P, do=P, lse=P, seg=None, scale=0.125, causal=1, dq=P, dk=P, dv=P,
                 B=1, H=2, Hkv=None, N=64, D=64, dtype=0):
    Hkv = H if Hkv is None else Hkv
    return lib.fa_bwd_noalloc(q, k, v, o, do, lse, seg, ctypes.c_float(scale), causal, dq, dk, dv, B, H,
                              Hkv, N, D, dtype, None)


def test_bwd_noalloc_refusals(lib):
    """The allocation-free backward refuses, before any HIP call, what fa_bwd
    refuses, and shapes whose workspace exceeds its static array."""
    import memory_efficient_attention_amd as fa
    assert _bwd_noalloc(lib, dq=None) == FA_ERR_NULL
    assert _bwd_noalloc(lib, D=80) == FA_ERR_HEAD_DIM
    assert _bwd_noalloc(lib, scale=0.0) == FA_ERR_SCALE
    # the largest row count that fits, and one more 256-byte block than fits
    # (256 bytes of flags, then two fp32 arrays of B * H * N, each rounded up to 256 bytes)
    rows = ((fa.FA_NOALLOC_MAX_BYTES - 256) // 2 // 256 * 256) // 4
    assert lib.fa_workspace_bytes(1, 1, rows, 64, 0, 1) <= fa.FA_NOALLOC_MAX_BYTES
    assert lib.fa_workspace_bytes(1, 1, rows + 64, 64, 0, 1) > fa.FA_NOALLOC_MAX_BYTES
    assert _bwd_noalloc(lib, B=1, H=1, N=rows + 64) == FA_ERR_SCRATCH
    assert _bwd_noalloc(lib, B=64, H=32, N=4096) == FA_ERR_SCRATCH


def test_first_failing_check_wins(lib):
    # a null pointer is reported before a bad shape, a bad shape before a bad dtype
    assert _fwd(lib, q=None, B=0, dtype=9) == FA_ERR_NULL
    assert _fwd(lib, B=0, D=80, dtype=9) == FA_ERR_SHAPE
    assert _fwd(lib, D=80, dtype=9) == FA_ERR_HEAD_DIM


def test_workspace_sizes(lib):
    ws = lib.fa_workspace_bytes
    assert ws(1, 32, 16384, 128, 0, 0) == 0                    # plain forward needs none
    assert ws(0, 1, 1, 64, 0, 1) == 0 and ws(1, 1, 1, 80, 0, 1) == 0
    assert ws(1, 1, 1, 96, 0, 1) == 256 + 2 * 256                # head_dim 96 is supported
    b1 = ws(1, 32, 8192, 128, 0, 1)
    b2 = ws(1, 32, 16384, 128, 0, 1)
    # O(N): two fp32 (B,H,N) arrays plus a 256-byte flag block
    assert b1 == 256 + 2 * 32 * 8192 * 4 and b2 == 256 + 2 * 32 * 16384 * 4
    s1 = ws(4, 32, 4096, 128, 1, 1)
    # + two range tables (int32 pairs) and two work lists (int32 quadruples)
    # per tile of 32
    assert s1 == 256 + 2 * 4 * 32 * 4096 * 4 + 2 * 4 * (4096 // 32) * (8 + 16)
    assert ws(1, 1, 100, 64, 1, 0) == 256 + 4 * 256           # each rounded to 256 B
    for n in (1000, 2000, 4000):
        assert ws(1, 8, 2 * n, 64, 1, 1) - 256 <= 2.01 * (ws(1, 8, n, 64, 1, 1) - 256)


def test_check_seg(lib):
    good = np.array([[0, 0, 1, 1, 1, 5], [2, 2, 2, 2, 2, 2]], dtype=np.int32)
    bad = np.array([[0, 0, 1, 0, 1, 5], [2, 2, 2, 2, 2, 2]], dtype=np.int32)
    assert lib.fa_check_seg(good.ctypes.data, 2, 6) == FA_OK
    assert lib.fa_check_seg(bad.ctypes.data, 2, 6) == FA_ERR_SEG
    # each row is checked on its own: a drop between rows is fine
    rows = np.array([[0, 1, 2], [0, 0, 1]], dtype=np.int32)
    assert lib.fa_check_seg(rows.ctypes.data, 2, 3) == FA_OK
    assert lib.fa_check_seg(None, 2, 3) == FA_ERR_NULL
    assert lib.fa_check_seg(rows.ctypes.data, 0, 3) == FA_ERR_SHAPE


def test_python_check_seg_raises():
    import memory_efficient_attention_amd as fa
    fa.fa_check_seg(np.zeros((1, 5), np.int32))
    with pytest.raises(fa.FaError) as e:
        fa.fa_check_seg(np.array([[1, 0]], np.int32))
    assert e.value.status == FA_ERR_SEG


def test_status_strings(lib):
    seen = set()
    for s in range(0, 12):
        txt = lib.fa_status_string(s).decode()
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 12
    assert lib.fa_status_string(1234).decode() == "unknown status"
    # the head-dim refusal names every supported head dim
    assert lib.fa_status_string(FA_ERR_HEAD_DIM).decode() == "head_dim must be 64, 96 or 128"


# ---------------------------------------------------------------- linear cross-entropy

def _lce_fwd(lib, h=P, w=P, t=P, nll=P, lse=P, tz=P, N=64, V=1000, D=256, dtype=0, ws=P, ws_bytes=1 << 30):
    lib.fa_lce_fwd.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                           ctypes.c_void_p]
    return lib.fa_lce_fwd(h, w, t, nll, lse, tz, N, V, D, dtype, ws, ws_bytes, None)


def _lce_bwd(lib, h=P, w=P, t=P, lse=P, g=P, dh=P, dw=P, N=64, V=1000, D=256, dtype=0, ws=P,
             ws_bytes=1 << 30):
    lib.fa_lce_bwd.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                           ctypes.c_void_p]
    return lib.fa_lce_bwd(h, w, t, lse, g, dh, dw, N, V, D, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), FA_ERR_NULL), (dict(t=None), FA_ERR_NULL), (dict(tz=None), FA_ERR_NULL),
    (dict(N=0), FA_ERR_SHAPE), (dict(V=0), FA_ERR_SHAPE), (dict(D=0), FA_ERR_SHAPE),
    (dict(D=320), FA_ERR_SHAPE), (dict(V=1 << 20, D=1024), FA_ERR_SHAPE),
    (dict(N=1 << 17), FA_ERR_SHAPE),
    (dict(dtype=1), FA_ERR_DTYPE), (dict(dtype=5), FA_ERR_DTYPE),
    (dict(h=P + 8), FA_ERR_ALIGN), (dict(nll=P + 2), FA_ERR_ALIGN),
    (dict(ws=None), FA_ERR_WORKSPACE), (dict(ws_bytes=64), FA_ERR_WORKSPACE), (dict(ws=P + 128), FA_ERR_ALIGN),
])
def test_lce_fwd_refusals(lib, kw, status):
    assert _lce_fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), FA_ERR_NULL), (dict(dh=None), FA_ERR_NULL), (dict(lse=None), FA_ERR_NULL),
    (dict(D=100), FA_ERR_SHAPE), (dict(dtype=1), FA_ERR_DTYPE),
    (dict(dw=P + 8), FA_ERR_ALIGN), (dict(g=P + 1), FA_ERR_ALIGN),
    (dict(ws=None), FA_ERR_WORKSPACE), (dict(ws_bytes=1024), FA_ERR_WORKSPACE),
])
def test_lce_bwd_refusals(lib, kw, status):
    assert _lce_bwd(lib, **kw) == status


def test_lce_workspace_sizes(lib):
    ws = lib.fa_lce_workspace_bytes
    ws.argtypes = [ctypes.c_int] * 4
    ws.restype = ctypes.c_size_t
    assert ws(8192, 151936, 4096, 0) == 594 * 8192 * 8       # per-tile (max, sum) pairs
    # one dZ chunk of 8192 vocabulary columns, plus the fp32 dh accumulator when
    # the vocabulary spans several chunks
    assert ws(8192, 151936, 4096, 1) == 8192 * 8192 * 2 + 8192 * 4096 * 4
    assert ws(100, 5000, 256, 1) == 100 * 8192 * 2
    assert ws(100, 5000, 255, 1) == 0 and ws(0, 5000, 256, 0) == 0


def test_python_binding_refuses_host_tensors():
    """The binding checks its tensors before touching the library: host
    (CPU) tensors are refused with a ValueError, never passed on as device
    pointers."""
    torch = pytest.importorskip("torch")
    import memory_efficient_attention_amd as fa
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_fwd(q, q, q)
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_bwd(q, q, q, q, q, torch.zeros(1, 2, 16))
    h = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_lce_fwd(h, h, torch.zeros(8, dtype=torch.int32))
