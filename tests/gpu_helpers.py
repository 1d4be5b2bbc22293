"""Shared helpers for the GPU parity tests: upload, run through the C ABI,
compare against the fp64 oracle with the stated bounds."""
from __future__ import annotations

import sys

import numpy as np

# Bounds (see the test docstrings): bf16 inputs: O max-abs <= max(1e-2, one bf16
# ulp of the exact value), dQ/dK/dV relative L2 <= 2e-2; fp32 inputs: O max-abs
# <= 1e-4 and relative L2 <= 1e-4.  LSE (internal check): 1e-3 / 1e-5, relative
# to |LSE| once that exceeds 10 (the kernels hold LSE in fp32, whose ulp alone
# passes 1e-5 above 128).
O_ABS = {"bf16": 1e-2, "fp32": 1e-4}
REL_L2 = {"bf16": 2e-2, "fp32": 1e-4}
LSE_ABS = {"bf16": 1e-3, "fp32": 1e-5}
LSE_SCALE_FROM = 10.0


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def upload(x: np.ndarray, dtype: str):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch_dtype(dtype))


def upload_seg(seg):
    import torch
    if seg is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).to("cuda")


def down(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = "O") -> float:
    err = np.abs(o_gpu - o_ref)
    if dtype == "bf16":
        bound = np.maximum(O_ABS["bf16"], bf16_ulp(o_ref))
    else:
        bound = np.full_like(o_ref, O_ABS["fp32"])
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over bound, worst err "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    if dtype == "bf16":
        # how many elements needed the one-ulp allowance, next to what rounding
        # the exact reference to bf16 alone costs on these inputs
        import workloads
        floor = np.abs(workloads.bf16_round(o_ref.astype(np.float32)).astype(np.float64) - o_ref).max()
        say(f"  {what}: max err {err.max():.3e}; {int((err > O_ABS['bf16']).sum())} elements used the "
            f"bf16-ulp allowance; bf16 rounding floor of the reference {floor:.3e}")
    return float(err.max())


def rel_l2(g: np.ndarray, r: np.ndarray) -> float:
    """||g - r|| / ||r|| over the whole tensor, with ||r|| floored at an RMS of
    1e-2 per element (about 1 % of the RMS gradient of unit-normal inputs) so
    that an exactly-zero reference (e.g. dK of a one-token sequence, where the
    GPU's fp32 cancellation of dP against D_i leaves ~1e-7) is judged on an
    absolute scale instead of dividing by ~0."""
    floor = 1e-2 * np.sqrt(r.size)
    return float(np.linalg.norm((g - r).ravel()) / max(np.linalg.norm(r.ravel()), floor))


def check_grad(g: np.ndarray, r: np.ndarray, dtype: str, what: str) -> float:
    e = rel_l2(g, r)
    assert e <= REL_L2[dtype], f"{what}: relative L2 {e:.3e} > {REL_L2[dtype]}"
    return e


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, dtype: str) -> float:
    err = np.abs(l_gpu - l_ref)
    bound = LSE_ABS[dtype] * np.maximum(1.0, np.abs(l_ref) / LSE_SCALE_FROM)
    bad = err > bound
    assert not bad.any(), (f"LSE: {int(bad.sum())} over bound, worst err {err.max():.3e} "
                           f"at |LSE| {np.abs(l_ref).ravel()[err.argmax()]:.3g}")
    return float(err.max())


def run_gpu(t: dict, seg, dtype: str, scale: float, causal: bool):
    """fa_fwd + fa_bwd through the C ABI; returns device tensors."""
    import torch
    import memory_efficient_attention_amd as fa
    q, k, v, do = (upload(t[n], dtype) for n in ("q", "k", "v", "do"))
    sg = upload_seg(seg)
    o, lse = fa.fa_fwd(q, k, v, sg, scale, causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, sg, scale, causal)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, seg=sg, o=o, lse=lse, dq=dq, dk=dk, dv=dv)
