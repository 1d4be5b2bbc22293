"""The autograd wrappers route through the same C-ABI calls: flash_attention's
gradients equal fa_bwd's on the same upstream gradient bit for bit (and the
oracle's within the usual bounds), and linear_cross_entropy's loss and
gradients equal fa_lce_fwd / fa_lce_bwd's for each reduction."""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_grad, check_o, down, say
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_attention_amd as fa
    fa.load_library()
    yield


@pytest.mark.parametrize("packed", [False, True])
def test_flash_attention_autograd(packed):
    import torch
    import memory_efficient_attention_amd as fa
    B, H, Hkv, N, D = 1, 4, 2, 300, 64
    say(f"flash_attention autograd B{B} H{H} Hkv{Hkv} N{N} D{D} packed={packed}")
    t = workloads.make_tensors(B, H, N, D, "bf16", 21, Hkv=Hkv)
    seg_np = workloads.random_segments(B, N, 21, max_len=90) if packed else None
    seg = None if seg_np is None else torch.from_numpy(seg_np).cuda()
    q, k, v = (torch.from_numpy(t[n]).cuda().bfloat16().requires_grad_() for n in ("q", "k", "v"))
    do = torch.from_numpy(t["do"]).cuda().bfloat16()
    scale = 1.0 / np.sqrt(D)
    out = fa.flash_attention(q, k, v, scale=scale, causal=True, segments=seg)
    out.backward(do)
    o2, lse2 = fa.fa_fwd(q.detach(), k.detach(), v.detach(), seg, scale, True)
    dq2, dk2, dv2 = fa.fa_bwd(q.detach(), k.detach(), v.detach(), o2, do, lse2, seg, scale, True)
    torch.cuda.synchronize()
    assert bool((out.detach() == o2).all())
    for name, a, b in (("dq", q.grad, dq2), ("dk", k.grad, dk2), ("dv", v.grad, dv2)):
        assert bool((a == b).all()), f"{name}: autograd differs from fa_bwd"
    o_r, lse_r = attention_forward(t["q"], t["k"], t["v"], seg_np, scale, True)
    g_r = attention_backward(t["q"], t["k"], t["v"], t["do"], seg_np, scale, True, o=o_r, lse=lse_r)
    pv_r, _ = attention_forward(t["q"], t["k"], np.abs(t["v"]), seg_np, scale, True)
    check_o(down(out), o_r, "bf16", pv_abs=pv_r)
    for name, g, r in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), g_r):
        check_grad(down(g), r, "bf16", name)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_linear_cross_entropy_autograd(reduction):
    import torch
    import memory_efficient_attention_amd as fa
    N, V, D = 200, 3000, 256
    say(f"linear_cross_entropy autograd N{N} V{V} D{D} reduction={reduction}")
    x = workloads.make_lce_inputs(N, V, D, 22)
    h = torch.from_numpy(x["h"]).cuda().bfloat16().requires_grad_()
    w = torch.from_numpy(x["w"]).cuda().bfloat16().requires_grad_()
    t = torch.from_numpy(x["targets"]).cuda()
    nll_t = fa.linear_cross_entropy(h, w, t)
    # the reduction is the caller's (torch here, in the test)
    loss = {"mean": lambda x: x.mean(), "sum": lambda x: x.sum(), "none": lambda x: x}[reduction](nll_t)
    if reduction == "none":
        g = torch.linspace(0.5, 1.5, N, device="cuda")
        loss.backward(g)
    else:
        loss.backward()
        g = torch.full((N,), 1.0 / N if reduction == "mean" else 1.0, device="cuda")
    nll, lse, _ = fa.fa_lce_fwd(h.detach(), w.detach(), t)
    dh, dw = fa.fa_lce_bwd(h.detach(), w.detach(), t, lse, g.float())
    torch.cuda.synchronize()
    want = {"mean": nll.mean(), "sum": nll.sum(), "none": nll}[reduction]
    assert bool((loss.detach() == want).all())
    assert bool((h.grad == dh).all()) and bool((w.grad == dw).all())
