"""HIP-graph capture of the entry points.

The calls make no allocation, memset or host synchronisation, so a caller can
capture them in a graph.  Each test captures fwd + bwd with caller-supplied
buffers, then replays the graph several times; before each replay it writes
new inputs into the captured buffers and runs eager work (including the
same calls eagerly) with a synchronisation in between, and every replay must
equal the eager result on the same inputs bit for bit (the kernels are
deterministic)."""
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


@pytest.mark.parametrize("packed", [False, True])
def test_attention_graph_replays_match_eager(packed):
    import torch
    import memory_efficient_attention_amd as fa
    from gpu_helpers import say
    B, H, Hkv, N, D = 2, 4, 2, 700, 128
    say(f"graph capture B{B} H{H} Hkv{Hkv} N{N} D{D} packed={packed}")
    g = torch.Generator(device="cuda").manual_seed(11)
    q, do = (torch.empty(B, H, N, D, device="cuda", dtype=torch.bfloat16) for _ in range(2))
    k, v = (torch.empty(B, Hkv, N, D, device="cuda", dtype=torch.bfloat16) for _ in range(2))
    seg = None
    if packed:
        seg = (torch.arange(N, device="cuda", dtype=torch.int32) // 97).repeat(B, 1).contiguous()
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty(B, H, N, device="cuda")
    ws = torch.empty(max(fa.fa_workspace_bytes(B, H, N, D, packed, True), 256), dtype=torch.uint8, device="cuda")

    def refill():
        for t in (q, k, v, do):
            t.copy_(torch.randn(t.shape, device="cuda", generator=g))

    def step():
        fa.fa_fwd(q, k, v, seg, None, True, out=o, lse=lse, workspace=ws)
        fa.fa_bwd(q, k, v, o, do, lse, seg, None, True, dq=dq, dk=dk, dv=dv, workspace=ws)

    refill()
    step()   # load code objects before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        refill()
        step()                                   # eager, same buffers
        torch.cuda.synchronize()
        want = [t.clone() for t in (o, lse, dq, dk, dv)]
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))                # the replay must overwrite everything
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), want):
            assert bool((got == ref).all()), f"replay {rep}: {name} differs from eager"


def test_loss_layer_graph_replays_match_eager():
    import torch
    import memory_efficient_attention_amd as fa
    from gpu_helpers import say
    N, V, D = 300, 20000, 256
    say(f"graph capture loss layer N{N} V{V} D{D}")
    g = torch.Generator(device="cuda").manual_seed(12)
    h = torch.empty(N, D, device="cuda", dtype=torch.bfloat16)
    w = torch.empty(V, D, device="cuda", dtype=torch.bfloat16)
    t = torch.empty(N, device="cuda", dtype=torch.int32)
    dn = torch.full((N,), 1.0 / N, device="cuda")
    lib = fa.load_library()
    wf, wb = fa.fa_lce_workspace_bytes(N, V, D, False), fa.fa_lce_workspace_bytes(N, V, D, True)
    wsf = torch.empty(wf, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(wb, dtype=torch.uint8, device="cuda")
    nll, lse, tz = (torch.empty(N, device="cuda") for _ in range(3))
    dh, dw = torch.empty_like(h), torch.empty_like(w)

    def refill():
        h.copy_(torch.randn(N, D, device="cuda", generator=g))
        w.copy_(torch.randn(V, D, device="cuda", generator=g) * D ** -0.5)
        t.copy_(torch.randint(0, V, (N,), device="cuda", generator=g, dtype=torch.int32))

    def step():
        st = torch.cuda.current_stream().cuda_stream
        assert lib.fa_lce_fwd(h.data_ptr(), w.data_ptr(), t.data_ptr(), nll.data_ptr(), lse.data_ptr(),
                              tz.data_ptr(), N, V, D, 0, wsf.data_ptr(), wf, st) == 0
        assert lib.fa_lce_bwd(h.data_ptr(), w.data_ptr(), t.data_ptr(), lse.data_ptr(), dn.data_ptr(),
                              dh.data_ptr(), dw.data_ptr(), N, V, D, 0, wsb.data_ptr(), wb, st) == 0

    refill()
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        refill()
        step()
        torch.cuda.synchronize()
        want = [x.clone() for x in (nll, lse, tz, dh, dw)]
        for x in (nll, lse, tz, dh, dw):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("nll", "lse", "tlogit", "dh", "dw"), (nll, lse, tz, dh, dw), want):
            assert bool((got == ref).all()), f"replay {rep}: {name} differs from eager"
