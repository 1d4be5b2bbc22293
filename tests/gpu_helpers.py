"""Shared helpers for the GPU parity tests: upload, run through the C ABI,
compare against the fp64 oracle with the stated bounds."""
from __future__ import annotations

import sys

import numpy as np

# Bounds (see the test docstrings): bf16 inputs: O max-abs <= 1e-2, or the bound
# of the method's bf16 roundings of P and O where that is larger (o_bound),
# dQ/dK/dV relative L2
# <= 2e-2 with no floor (an exactly-zero reference takes the absolute bound of
# zero_grad_bounds); fp32 inputs: O max-abs <= 1e-4 and relative L2 <= 1e-4.
# LSE (internal check): 1e-3 / 1e-5, relative to |LSE| once that exceeds 10 (the kernels hold LSE in fp32, whose ulp alone
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


def o_bound(o_ref: np.ndarray, dtype: str, pv_abs=None) -> np.ndarray:
    """Per-element bound on |O_gpu - O_ref|.  fp32: 1e-4.  bf16: the stated
    1e-2, or where the method's own roundings can exceed it, their bound:
    the kernels round P to bf16 (unit roundoff 2^-8) before the P V product,
    which moves O_id by at most 2^-8 sum_j P_ij |v_jd| = 2^-8 (P|V|)_id
    (`pv_abs`, the oracle's attention output for |V|), and then round O to
    bf16, half an ulp of the value.  fp32 accumulation adds ~1e-6."""
    if dtype != "bf16":
        return np.full_like(o_ref, O_ABS["fp32"])
    assert pv_abs is not None, "bf16 O checks need the oracle's P|V| (pv_abs)"
    ep = 2.0 ** -8 * pv_abs
    return np.maximum(O_ABS["bf16"], ep + 0.5 * bf16_ulp(np.abs(o_ref) + ep) + 1e-5)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = "O", pv_abs=None) -> float:
    err = np.abs(o_gpu - o_ref)
    bound = o_bound(o_ref, dtype, pv_abs)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over bound, worst err "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    if dtype == "bf16":
        # how many elements needed the rounding allowance, next to what rounding
        # the exact reference to bf16 alone costs on these inputs
        import workloads
        floor = np.abs(workloads.bf16_round(o_ref.astype(np.float32)).astype(np.float64) - o_ref).max()
        say(f"  {what}: max err {err.max():.3e}; {int((err > O_ABS['bf16']).sum())} elements used the "
            f"bf16 rounding allowance; bf16 rounding floor of the reference {floor:.3e}")
    return float(err.max())


def rel_l2(g: np.ndarray, r: np.ndarray) -> float:
    """||g - r|| / ||r|| over the whole tensor, in fp64, with no floor."""
    return float(np.linalg.norm((g - r).ravel()) / np.linalg.norm(r.ravel()))


# unit roundoff of the fp32 accumulation every kernel uses
U32 = 2.0 ** -24


def zero_grad_bounds(out: dict, scale: float) -> dict:
    """Element-wise bounds on dQ and dK where every row sees only itself
    (N = 1, or every segment one token long), so that their exact values are
    0.  There P_ii = 1 and dS_ii = dP_ii - D_i = dO_i . v_i - dO_i . O_i with
    O_i = v_i, i.e. two fp32 dot products of the same D products summed in
    different orders: |dS_ii| <= 2 D u sum_d |dO_id v_id| (u = 2^-24, the
    usual bound for a D-term fp32 sum; rounding dS to bf16 only scales it by
    1 + 2^-8).  Then |dQ_id| <= scale |dS_ii| |k_id| and |dK_jd| <= scale
    sum over the query heads h of j's group of |dS_hjj| |q_hjd|.  A factor 2
    covers P_ii = 1 within a few fp32 ulps and the rounding of the products."""
    q, k, v, do = (down(out[n]) for n in ("q", "k", "v", "do"))
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    vq = np.repeat(v, G, axis=1)                      # each query head's key/value head
    ds = 2.0 * D * U32 * np.abs(do * vq).sum(axis=-1, keepdims=True)   # (B, H, N, 1)
    dq = 2.0 * scale * ds * np.abs(np.repeat(k, G, axis=1))
    dk = 2.0 * scale * (ds * np.abs(q)).reshape(B, Hkv, G, N, D).sum(axis=2)
    return {"dq": dq, "dk": dk}


def check_grad(g: np.ndarray, r: np.ndarray, dtype: str, what: str, zero_bound=None) -> float:
    """Relative L2 <= REL_L2[dtype].  Where the caller knows the exact value
    is zero by construction (every row sees only itself, see
    zero_grad_bounds), it passes `zero_bound` (an array, or a callable that
    returns one): there is no relative error to take then (the fp64 oracle
    itself leaves ~1e-17 of rounding), so the reference must be zero to fp64
    rounding and the GPU value within that absolute bound, element-wise."""
    if zero_bound is not None:
        if callable(zero_bound):
            zero_bound = zero_bound()
        assert np.abs(r).max() <= 1e-12, f"{what}: the reference is not zero ({np.abs(r).max():.3e})"
        bad = np.abs(g) > zero_bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements above the fp32 cancellation bound, "
                               f"worst |g| {np.abs(g).max():.3e}")
        return float(np.abs(g).max())
    e = rel_l2(g, r)
    assert e <= REL_L2[dtype], f"{what}: relative L2 {e:.3e} > {REL_L2[dtype]}"
    return e


def sees_only_itself(out: dict) -> bool:
    """Every row's only visible key is itself: N = 1, or every segment one
    token long.  dQ and dK are then exactly zero."""
    N = out["q"].shape[2]
    if N == 1:
        return True
    seg = out["seg"]
    if seg is None:
        return False
    s = seg.detach().cpu().numpy()
    return bool((s[:, 1:] != s[:, :-1]).all())


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
    return dict(q=q, k=k, v=v, do=do, seg=sg, o=o, lse=lse, dq=dq, dk=dk, dv=dv, scale=scale)
