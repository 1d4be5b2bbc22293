"""The allocation-free backward (fa_bwd_noalloc) against fa_bwd (collected last:
its name sorts after every other test file).

fa_bwd_noalloc runs fa_bwd's kernels on a static workspace inside the
library, so on the same inputs its outputs must equal fa_bwd's bit for bit
(and hence meet the oracle bounds fa_bwd meets).  Two calls in a row, the
second smaller than the first, show that a call does not depend on what the
previous one left in the shared array; both are compared, and the second is
also checked against the oracle.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import check_grad, down, say, upload, upload_seg
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


def _case(B, H, Hkv, N, D, dtype, packed, seed):
    import torch
    import memory_efficient_attention_amd as fa
    say(f"no-alloc backward B{B} H{H} Hkv{Hkv} N{N} D{D} {dtype} packed={packed} seed {seed}")
    t = workloads.make_tensors(B, H, N, D, dtype, seed, Hkv=Hkv)
    seg = workloads.random_segments(B, N, seed, max_len=N // 3) if packed else None
    q, k, v, do = (upload(t[n], dtype) for n in ("q", "k", "v", "do"))
    sg = upload_seg(seg)
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fa_fwd(q, k, v, sg, scale, True)
    ref = fa.fa_bwd(q, k, v, o, do, lse, sg, scale, True)
    out = tuple(torch.full_like(x, float("nan")) for x in ref)
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, sg, scale, True, dq=out[0], dk=out[1], dv=out[2])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), out, ref):
        assert bool((a == b).all()), f"{name}: fa_bwd_noalloc differs from fa_bwd"
    return t, seg, scale, out


def test_two_calls_second_smaller_match_fa_bwd():
    _case(2, 4, 2, 1000, 128, "bf16", True, 301)
    t, seg, scale, out = _case(1, 2, 2, 300, 64, "bf16", False, 302)
    o_r, lse_r = attention_forward(t["q"], t["k"], t["v"], seg, scale, True)
    g_r = attention_backward(t["q"], t["k"], t["v"], t["do"], seg, scale, True, o=o_r, lse=lse_r)
    for name, g, r in zip(("dq", "dk", "dv"), out, g_r):
        check_grad(down(g), r, "bf16", name)


def test_too_large_is_refused():
    import torch
    import memory_efficient_attention_amd as fa
    B, H, N, D = 1, 1, ((fa.FA_NOALLOC_MAX_BYTES - 256) // 2 // 256 * 256) // 4 + 64, 64
    say(f"no-alloc backward refusal B{B} H{H} N{N} D{D}")
    x = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_noalloc(x, x, x, x, x, lse, None, 0.125, True, dq=x, dk=x, dv=x)
    assert e.value.status == fa.FA_ERR_SCRATCH


def test_graph_capture_of_the_allocation_free_backward():
    """The callers it is for: a dense causal step (fa_fwd needs no workspace
    there) with fa_bwd_noalloc, captured in a HIP graph with no buffer but
    the inputs and outputs; every replay equals the eager step bitwise, with
    new inputs and eager work between replays."""
    import torch
    import memory_efficient_attention_amd as fa
    B, H, N, D = 1, 4, 600, 128
    say(f"graph capture of fa_fwd + fa_bwd_noalloc B{B} H{H} N{N} D{D}")
    g = torch.Generator(device="cuda").manual_seed(13)
    q, k, v, do = (torch.empty(B, H, N, D, device="cuda", dtype=torch.bfloat16) for _ in range(4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(B, H, N, device="cuda")

    def refill():
        for t in (q, k, v, do):
            t.copy_(torch.randn(t.shape, device="cuda", generator=g))

    def step():
        fa.fa_fwd(q, k, v, None, None, True, out=o, lse=lse)
        fa.fa_bwd_noalloc(q, k, v, o, do, lse, None, None, True, dq=dq, dk=dk, dv=dv)

    refill()
    step()   # code objects loaded and the array's address looked up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        refill()
        step()
        torch.cuda.synchronize()
        want = [t.clone() for t in (o, lse, dq, dk, dv)]
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), want):
            assert bool((got == ref).all()), f"replay {rep}: {name} differs from eager"
