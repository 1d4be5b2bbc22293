"""O(N) memory, measured on the device.

The library never allocates: with every output and the workspace supplied
by the caller, fa_fwd + fa_bwd and fa_lce_fwd + fa_lce_bwd must not raise
the device's allocated bytes at all, and the workspace they ask for is
O(B*H*N) for attention (O(N*chunk) for the loss), far below the (N, N)
score matrix or the (N, V) logits the fused kernels avoid.  Values are
random (memory does not depend on them)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_attention_amd as fa
    fa.load_library()
    yield


def _peak_extra(fn):
    import torch
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fn()
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() - base


def test_attention_allocates_nothing_and_workspace_is_linear():
    import torch
    import memory_efficient_attention_amd as fa
    from gpu_helpers import say
    B, H, N, D = 1, 32, 16384, 128
    g = torch.Generator(device="cuda").manual_seed(3)
    q, k, v, do = (torch.randn(B, H, N, D, device="cuda", generator=g).bfloat16() for _ in range(4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(B, H, N, device="cuda")
    wf = fa.fa_workspace_bytes(B, H, N, D, False, False)
    wb = fa.fa_workspace_bytes(B, H, N, D, False, True)
    ws = torch.empty(max(wf, wb, 256), dtype=torch.uint8, device="cuda")

    def step():
        fa.fa_fwd(q, k, v, None, None, True, out=o, lse=lse, workspace=ws)
        fa.fa_bwd(q, k, v, o, do, lse, None, None, True, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()   # first call loads code objects
    extra = _peak_extra(step)
    tensor = B * H * N * D * 2
    say(f"  workspace fwd {wf} B, bwd {wb} B; one tensor {tensor} B; (N, N) bf16 scores per head "
        f"{N * N * 2} B; extra device bytes during the step {extra}")
    assert extra == 0
    assert wb <= 256 + 2 * B * H * N * 4          # two fp32 rows per (b, h, n)
    assert wb < tensor // 16


def test_loss_layer_allocates_nothing_and_workspace_is_far_below_logits():
    import torch
    import memory_efficient_attention_amd as fa
    from gpu_helpers import say
    N, V, D = 8192, 151936, 4096
    g = torch.Generator(device="cuda").manual_seed(4)
    h = torch.randn(N, D, device="cuda", generator=g).bfloat16()
    w = (torch.randn(V, D, device="cuda", generator=g) * D ** -0.5).bfloat16()
    t = torch.randint(0, V, (N,), device="cuda", generator=g, dtype=torch.int32)
    dn = torch.full((N,), 1.0 / N, device="cuda")
    wf = fa.fa_lce_workspace_bytes(N, V, D, False)
    wb = fa.fa_lce_workspace_bytes(N, V, D, True)
    wsf = torch.empty(wf, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(wb, dtype=torch.uint8, device="cuda")
    lib = fa.load_library()
    nll, lse, tz = (torch.empty(N, device="cuda") for _ in range(3))
    dh, dw = torch.empty_like(h), torch.empty_like(w)
    st = torch.cuda.current_stream().cuda_stream

    def step():
        assert lib.fa_lce_fwd(h.data_ptr(), w.data_ptr(), t.data_ptr(), nll.data_ptr(), lse.data_ptr(),
                              tz.data_ptr(), N, V, D, 0, wsf.data_ptr(), wf, st) == 0
        assert lib.fa_lce_bwd(h.data_ptr(), w.data_ptr(), t.data_ptr(), lse.data_ptr(), dn.data_ptr(),
                              dh.data_ptr(), dw.data_ptr(), N, V, D, 0, wsb.data_ptr(), wb, st) == 0

    step()
    extra = _peak_extra(step)
    logits = N * V * 2
    say(f"  loss workspace fwd {wf} B, bwd {wb} B; bf16 logits {logits} B; extra device bytes {extra}")
    assert extra == 0
    assert wf < logits // 50 and wb < logits // 8


def test_caller_workspace_is_checked_not_replaced():
    """A caller that passes a workspace gets no allocation: one too small, or
    in host memory, is refused instead of silently replaced."""
    import torch
    import memory_efficient_attention_amd as fa
    B, H, N, D = 1, 2, 300, 64
    q, k, v, do = (torch.randn(B, H, N, D, device="cuda").bfloat16() for _ in range(4))
    seg = (torch.arange(N, device="cuda", dtype=torch.int32) // 50).reshape(1, N).contiguous()
    need = fa.fa_workspace_bytes(B, H, N, D, True, True)
    o, lse = fa.fa_fwd(q, k, v, seg)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="bytes"):
        fa.fa_bwd(q, k, v, o, do, lse, seg, workspace=small)
    with pytest.raises(ValueError, match="workspace is on"):
        fa.fa_bwd(q, k, v, o, do, lse, seg, workspace=torch.empty(need, dtype=torch.uint8))
    exact = torch.empty(need, dtype=torch.uint8, device="cuda")
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, seg, workspace=exact)
    dq2, dk2, dv2 = fa.fa_bwd(q, k, v, o, do, lse, seg)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert bool((a == b).all())
