"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Bounds, per tensor:
* bf16 inputs: |O - O_ref| <= max(1e-2, one bf16 ulp of O_ref) element-wise
  (1e-2 is the stated bound; the ulp allowance covers the bf16 rounding of
  the output itself, which alone can exceed 1e-2 where |O| >= 2), and
  relative L2 error <= 2e-2 for dQ, dK and dV;
* fp32 inputs: O max-abs <= 1e-4 and relative L2 <= 1e-4;
* LSE max-abs <= 1e-3 (bf16) / 1e-5 (fp32).

Small shapes run the whole oracle; they span several tiles and a ragged tail
(N = 1, 17, 129, 255, 257, 300) in every masking mode.  The five workloads
run at full size on the GPU; the oracle then checks whole sampled heads,
sampled rows, or (for very long packed rows) whole segments run alone, which
equals the packed row by the oracle's own pinned invariant.  Full-size outputs
are also checked against identities that need no oracle.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import (check_grad, check_lse, check_o, down, run_gpu, say, sees_only_itself, upload,
                         upload_seg, zero_grad_bounds)
from oracle import attention_backward, attention_forward, attention_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_efficient_attention_amd as fa
    fa.load_library()        # raises if the HIP library is missing: no fallback
    torch.manual_seed(0)
    yield


def _oracle_full(t, seg, scale, causal):
    o, lse = attention_forward(t["q"], t["k"], t["v"], seg, scale, causal)
    pv, _ = attention_forward(t["q"], t["k"], np.abs(t["v"]), seg, scale, causal)   # P|V|, for o_bound
    dq, dk, dv = attention_backward(t["q"], t["k"], t["v"], t["do"], seg, scale, causal, o=o, lse=lse)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, pv=pv)


def _compare(out, ref, dtype, sl=(slice(None),), tag=""):
    """Compare GPU outputs (device tensors) against oracle arrays on index `sl`."""
    o = down(out["o"][sl])
    check_o(o, ref["o"], dtype, f"O{tag}", ref["pv"])
    check_lse(down(out["lse"][sl]), ref["lse"], dtype)
    # dQ and dK are exactly zero where every row sees only itself: checked
    # against the absolute bound of the fp32 cancellation instead
    zero = sees_only_itself(out)

    def zb(n):
        return (lambda: zero_grad_bounds(out, out["scale"])[n][sl]) if zero and n != "dv" else None
    errs = [check_grad(down(out[n][sl]), ref[n], dtype, f"{n}{tag}", zero_bound=zb(n)) for n in ("dq", "dk", "dv")]
    return errs


# ---------------------------------------------------------------- small shapes

# N = 512 and 768 (whole 256-row workgroups, grids far below one per CU) take
# the mirrored block order in dense causal calls
SHAPES = [(1, 2, 1, 64), (1, 1, 17, 64), (2, 2, 255, 128), (1, 2, 257, 64), (1, 3, 300, 128),
          (2, 1, 129, 128), (1, 2, 200, 96), (2, 1, 65, 96), (1, 2, 512, 64), (2, 3, 768, 128),
          (1, 2, 512, 96)]
MODES = {"causal": (False, True), "packed": (True, True), "packed_bidir": (True, False),
         "full": (False, False)}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,H,N,D", SHAPES)
def test_small_shapes(B, H, N, D, dtype, mode):
    packed, causal = MODES[mode]
    seed = 1000 + 7 * N + D + B
    say(f"small case B{B} H{H} N{N} D{D} {dtype} {mode} seed {seed}")
    t = workloads.make_tensors(B, H, N, D, dtype, seed)
    seg = workloads.random_segments(B, N, seed, max_len=max(1, N // 4)) if packed else None
    scale = 1.0 / np.sqrt(D)
    out = run_gpu(t, seg, dtype, scale, causal)
    ref = _oracle_full(t, seg, scale, causal)
    _compare(out, ref, dtype)


# group sizes 2 and 4 take the two-team dK/dV workgroups in dense bf16 calls;
# the group of 3 takes the single-team one.  N a multiple of 128 (256 for
# the forward and dQ) takes the mirrored block order in dense causal calls.
GQA_SHAPES = [(1, 4, 2, 129, 64), (2, 4, 1, 257, 128), (1, 6, 3, 200, 128), (1, 4, 2, 150, 96),
              (1, 6, 2, 160, 128), (1, 4, 2, 512, 128), (1, 4, 2, 384, 64), (1, 6, 3, 256, 128)]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,H,Hkv,N,D", GQA_SHAPES)
def test_grouped_query_heads(B, H, Hkv, N, D, dtype, mode):
    """K/V with fewer heads than Q: query head h reads key/value head
    h // (H / Hkv), and dK/dV of a key/value head sum over its query heads."""
    packed, causal = MODES[mode]
    seed = 2000 + 7 * N + D + H + Hkv
    say(f"grouped heads B{B} H{H} Hkv{Hkv} N{N} D{D} {dtype} {mode} seed {seed}")
    t = workloads.make_tensors(B, H, N, D, dtype, seed, Hkv=Hkv)
    seg = workloads.random_segments(B, N, seed, max_len=max(1, N // 4)) if packed else None
    scale = 1.0 / np.sqrt(D)
    out = run_gpu(t, seg, dtype, scale, causal)
    assert tuple(out["dk"].shape) == (B, Hkv, N, D)
    _compare(out, _oracle_full(t, seg, scale, causal), dtype)


def test_short_segments_many_tiles():
    """Segments of 1..5 tokens: nearly every tile pair is cross-segment."""
    B, H, N, D = 2, 2, 700, 128
    say("short segments B2 H2 N700 D128 bf16")
    t = workloads.make_tensors(B, H, N, D, "bf16", 77)
    seg = workloads.random_segments(B, N, 77, max_len=5)
    for causal in (True, False):
        out = run_gpu(t, seg, "bf16", 0.09, causal)
        _compare(out, _oracle_full(t, seg, 0.09, causal), "bf16")


@pytest.mark.parametrize("offset", [1000, -5000])
def test_segment_ids_need_not_start_at_zero(offset):
    """Ids are compared for equality and order only; any non-decreasing ids
    work, negative ones included."""
    B, H, N, D = 1, 2, 200, 64
    say(f"offset segment ids B1 H2 N200 D64, offset {offset}")
    t = workloads.make_tensors(B, H, N, D, "bf16", 78)
    seg = workloads.random_segments(B, N, 78, max_len=50) * 3 + offset
    out = run_gpu(t, seg, "bf16", 0.125, True)
    _compare(out, _oracle_full(t, seg, 0.125, True), "bf16")


@pytest.mark.parametrize("mode", ["causal", "packed"])
def test_many_short_sequences(mode):
    """A large batch of short rows: thousands of one-tile workgroups, each
    row's tail inside its only tile."""
    B, H, N, D = 48, 8, 45, 64
    packed, causal = MODES[mode]
    say(f"many short rows B{B} H{H} N{N} D{D} bf16 {mode}")
    t = workloads.make_tensors(B, H, N, D, "bf16", 80)
    seg = workloads.random_segments(B, N, 80, max_len=12) if packed else None
    out = run_gpu(t, seg, "bf16", 0.125, causal)
    _compare(out, _oracle_full(t, seg, 0.125, causal), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_rising_and_falling_scores(D, dtype):
    """Scores that climb steeply along the keys move every row's softmax
    reference again on nearly every key tile (the rare rescale path); scores
    that fall keep the first tile's reference and underflow later tiles.

    The forward outputs are checked in both dtypes.  With softmax this sharp,
    P is one-hot to bf16 precision and dS = P (dP - D_i) is dominated by the
    cancellation of dP against D_i, which the method takes from the stored
    (bf16-rounded) O; in bf16 that difference is rounding noise on both
    sides, so dQ and dK are checked in fp32 only and dV (no D_i term) in
    both."""
    B, H, N = 1, 2, 300
    say(f"rising/falling scores B1 H2 N300 D{D} {dtype}")
    t = workloads.make_tensors(B, H, N, D, dtype, 79)
    ramp = (np.arange(N) / N * 8.0)[:, None] * np.ones((1, D))
    t["q"] = t["q"] * 0.25 + 2.0
    t["k"] = t["k"] * 0.25 + np.stack([ramp, ramp[::-1]])[None]   # head 0 rises, head 1 falls
    if dtype == "bf16":
        t = {n: workloads.bf16_round(x) for n, x in t.items()}
    scale = 1.0 / np.sqrt(D)
    seg = workloads.random_segments(B, N, 79, max_len=120)
    grads = ("dq", "dk", "dv") if dtype == "fp32" else ("dv",)
    for sg in (None, seg):
        out = run_gpu(t, sg, dtype, scale, True)
        ref = _oracle_full(t, sg, scale, True)
        check_o(down(out["o"]), ref["o"], dtype, pv_abs=ref["pv"])
        check_lse(down(out["lse"]), ref["lse"], dtype)
        for n in grads:
            check_grad(down(out[n]), ref[n], dtype, n)


def _sweep_cases(n=32, seed=4242):
    """A fixed, seeded list of small mixed configurations: batch, heads,
    group size, odd and whole-tile lengths, every head dim, both dtypes and
    every masking mode, with segment lengths from 1 token to the whole row."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 3, 4]))
        N = int(rng.choice([int(rng.integers(1, 600)), 128 * int(rng.integers(1, 5))]))
        cases.append(dict(B=int(rng.integers(1, 3)), H=Hkv * G, Hkv=Hkv, N=N, D=int(rng.choice([64, 96, 128])),
                          dtype=str(rng.choice(["bf16", "fp32"])), mode=str(rng.choice(list(MODES))),
                          max_len=int(rng.choice([1, 7, 60, N])), seed=5000 + i))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "B{B}H{H}Hkv{Hkv}N{N}D{D}{dtype}{mode}L{max_len}".format(**c))
def test_seeded_sweep(case):
    """Mixed small configurations against the full oracle."""
    c = case
    packed, causal = MODES[c["mode"]]
    say(f"sweep {c}")
    t = workloads.make_tensors(c["B"], c["H"], c["N"], c["D"], c["dtype"], c["seed"], Hkv=c["Hkv"])
    seg = workloads.random_segments(c["B"], c["N"], c["seed"], max_len=c["max_len"]) if packed else None
    scale = 1.0 / np.sqrt(c["D"])
    out = run_gpu(t, seg, c["dtype"], scale, causal)
    _compare(out, _oracle_full(t, seg, scale, causal), c["dtype"])


def _wide_cases(n=64, seed=777):
    """A second seeded list, wider than the first: up to 16 heads and groups
    of 8, lengths up to 1100 (ragged, whole 64-key tiles and 256-row
    workgroups +-2), segments of 1, 2, 7, 33, 64, 65 or 200 tokens or the
    whole row, softmax scales of 0.5, 1 and 2 times 1/sqrt(D), and, for bf16,
    queries 3 or 6 times larger (scores up to 12 times steeper)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 3, 4]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        while Hkv * G > 16:
            G //= 2
        N = max(1, int(rng.choice([int(rng.integers(1, 1100)), 64 * int(rng.integers(1, 17)),
                                   256 * int(rng.integers(1, 5)) + int(rng.integers(-2, 3))])))
        dtype = str(rng.choice(["bf16", "bf16", "fp32"]))
        cases.append(dict(B=int(rng.integers(1, 3)), H=Hkv * G, Hkv=Hkv, N=N, D=int(rng.choice([64, 96, 128])),
                          dtype=dtype, mode=str(rng.choice(list(MODES))),
                          max_len=int(rng.choice([1, 2, 7, 33, 64, 65, 200, N])),
                          qmul=float(rng.choice([1.0, 3.0, 6.0])) if dtype == "bf16" else 1.0,
                          scale_mul=float(rng.choice([0.5, 1.0, 2.0])), seed=90000 + i))
    return cases


@pytest.mark.parametrize("case", _wide_cases(),
                         ids=lambda c: "B{B}H{H}Hkv{Hkv}N{N}D{D}{dtype}{mode}L{max_len}q{qmul:g}s{scale_mul:g}".format(**c))
def test_seeded_wide_sweep(case):
    """The wider mixed configurations against the full oracle.  Where the
    scores are steeper than 1.5 times the usual scale in bf16, dQ and dK are
    not compared (the reading of test_rising_and_falling_scores: dS is then
    rounding noise of dP - D_i on both sides); O, LSE and dV are."""
    c = case
    packed, causal = MODES[c["mode"]]
    say(f"wide sweep {c}")
    t = workloads.make_tensors(c["B"], c["H"], c["N"], c["D"], c["dtype"], c["seed"], Hkv=c["Hkv"])
    if c["qmul"] != 1.0:
        t["q"] = workloads.bf16_round(t["q"] * c["qmul"])
    seg = workloads.random_segments(c["B"], c["N"], c["seed"], max_len=c["max_len"]) if packed else None
    scale = c["scale_mul"] / np.sqrt(c["D"])
    out = run_gpu(t, seg, c["dtype"], scale, causal)
    ref = _oracle_full(t, seg, scale, causal)
    if c["dtype"] == "bf16" and c["qmul"] * c["scale_mul"] > 1.5:
        check_o(down(out["o"]), ref["o"], "bf16", pv_abs=ref["pv"])
        check_lse(down(out["lse"]), ref["lse"], "bf16")
        check_grad(down(out["dv"]), ref["dv"], "bf16", "dv")
    else:
        _compare(out, ref, c["dtype"])


# ---------------------------------------------------------------- the workloads

def test_tiny_fp32_one_segment():
    w = workloads.get("tiny_causal_fp32")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    seg = w.seg()
    ref = _oracle_full(t, seg, w.scale, True)
    out = run_gpu(t, seg, w.dtype, w.scale, True)
    _compare(out, ref, w.dtype)
    plain = run_gpu(t, None, w.dtype, w.scale, True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((out[n] == plain[n]).all()), f"{n}: one-segment packed != causal"


def test_causal_2k_full_oracle():
    w = workloads.get("causal_2k")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    out = run_gpu(t, None, w.dtype, w.scale, True)
    ref = _oracle_full(t, None, w.scale, True)
    errs = _compare(out, ref, w.dtype)
    say(f"  rel-L2 dq/dk/dv {errs}")
    again = run_gpu(t, None, w.dtype, w.scale, True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((out[n] == again[n]).all()), f"{n} differs between identical runs"


def _seg_sums(x, seg):
    """Per-segment sums over tokens of x (B,H,N,D), and of |x|, in fp64."""
    import torch
    B, H, N, D = x.shape
    xs = x.to(torch.float64)
    ids = torch.zeros((B, N), dtype=torch.int64, device=x.device) if seg is None else seg.to(torch.int64)
    ids = ids - ids[:, :1]
    nseg = int(ids.max().item()) + 1
    sums = torch.zeros((B, H, nseg, D), dtype=torch.float64, device=x.device)
    mags = torch.zeros_like(sums)
    for b in range(B):
        sums[b].index_add_(1, ids[b], xs[b])
        mags[b].index_add_(1, ids[b], xs[b].abs())
    return sums, mags


def _invariants(out, tol=1e-2, tol_dk=0.1):
    """Identities of exact attention that hold at any size (no oracle):
    per segment sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i; per head
    sum_i q_i . dQ_i = sum_j k_j . dK_j.

    Bounds are relative to the sum of magnitudes.  sum dK = 0 rests on each
    row of dS summing to zero; with dS rounded to bf16 and D_i taken from the
    bf16-stored O, a row sums to O(2^-9 |D_i|) instead, which on segments of a
    few tokens reaches a few percent of sum |dK|; tol_dk = 0.1 still fails any
    structural error (a missed or extra tile), which gives ratios of order 1."""
    seg = out["seg"]
    B, H = out["q"].shape[:2]
    Hkv = out["k"].shape[1]
    dk_s, dk_m = _seg_sums(out["dk"], seg)
    assert bool((dk_s.abs() <= tol_dk * dk_m + 1e-6).all()), \
        f"sum dK per segment: worst {(dk_s.abs() / (dk_m + 1e-30)).max().item():.3e}"
    dv_s, dv_m = _seg_sums(out["dv"], seg)
    do_s, _ = _seg_sums(out["do"], seg)
    do_s = do_s.reshape(B, Hkv, H // Hkv, *do_s.shape[2:]).sum(dim=2)   # a group's query heads
    assert bool(((dv_s - do_s).abs() <= tol * dv_m + 1e-6).all()), "sum dV != sum dO per segment"
    qdq = (out["q"].double() * out["dq"].double()).sum(dim=(2, 3))
    lhs = qdq.reshape(B, Hkv, H // Hkv).sum(dim=2)
    rhs = (out["k"].double() * out["dk"].double()).sum(dim=(2, 3))
    mag = (out["q"].double() * out["dq"].double()).abs().sum(dim=(2, 3)).reshape(B, Hkv, -1).sum(dim=2)
    assert bool(((lhs - rhs).abs() <= tol * mag).all()), "sum q.dQ != sum k.dK"


def test_packed_short_examples_4k():
    w = workloads.get("packed_short_4k")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    seg = w.seg()
    out = run_gpu(t, seg, w.dtype, w.scale, True)
    for b, h in [(0, 0), (1, 17), (3, 31)]:
        say(f"  oracle head b{b} h{h}")
        tb = {n: t[n][b:b + 1, h:h + 1] for n in t}
        ref = _oracle_full(tb, seg[b:b + 1], w.scale, True)
        _compare(out, ref, w.dtype, (slice(b, b + 1), slice(h, h + 1)), f"[b{b} h{h}]")
    _invariants(out)


def test_causal_16k():
    w = workloads.get("causal_16k")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    out = run_gpu(t, None, w.dtype, w.scale, True)
    b, h = 0, 5
    say(f"  oracle head b{b} h{h}")
    tb = {n: t[n][b:b + 1, h:h + 1] for n in t}
    ref = _oracle_full(tb, None, w.scale, True)
    _compare(out, ref, w.dtype, (slice(b, b + 1), slice(h, h + 1)), f"[b{b} h{h}]")
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 16383], rng.integers(0, w.N, 27)]))
    o_all, lse_all = down(out["o"]), down(out["lse"])
    for hh in range(w.H):
        o_r, l_r = attention_rows(t["q"][0, hh], t["k"][0, hh], t["v"][0, hh], rows, None, w.scale, True)
        pv_r, _ = attention_rows(t["q"][0, hh], t["k"][0, hh], np.abs(t["v"][0, hh]), rows, None, w.scale, True)
        check_o(o_all[0, hh, rows], o_r, w.dtype, f"O rows h{hh}", pv_r)
        check_lse(lse_all[0, hh, rows], l_r, w.dtype)
    _invariants(out)


def test_single_segment_8k_bitwise_equals_causal():
    w = workloads.get("single_segment_8k")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    packed = run_gpu(t, w.seg(), w.dtype, w.scale, True)
    causal = run_gpu(t, None, w.dtype, w.scale, True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((packed[n] == causal[n]).all()), f"{n}: single-segment packed != causal"
    rows = np.array([0, 5, 100, 4097, 8191])
    o_r, l_r = attention_rows(t["q"][0, 3], t["k"][0, 3], t["v"][0, 3], rows, None, w.scale, True)
    pv_r, _ = attention_rows(t["q"][0, 3], t["k"][0, 3], np.abs(t["v"][0, 3]), rows, None, w.scale, True)
    check_o(down(packed["o"][0, 3, rows]), o_r, w.dtype, pv_abs=pv_r)
    check_lse(down(packed["lse"][0, 3, rows]), l_r, w.dtype)


@pytest.mark.parametrize("H,N", [(32, 2048), (32, 4096)])
def test_single_segment_bitwise_equals_causal_mirrored(H, N):
    """Dense causal grids of one (2k) or two (4k) rounds of the chip's CUs
    take the mirrored block order; the packed path never does.  Both must
    agree to the bit, since every row is walked in the same order."""
    w = workloads.get("causal_2k").with_(H=H, N=N)
    say(f"B1 H{H} N{N} D128 bf16 as one segment and as plain causal")
    t = w.tensors()
    seg = np.zeros((w.B, w.N), dtype=np.int32)
    packed = run_gpu(t, seg, w.dtype, w.scale, True)
    causal = run_gpu(t, None, w.dtype, w.scale, True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((packed[n] == causal[n]).all()), f"{n}: single-segment packed != causal"


@pytest.mark.parametrize("H,Hkv,N,D", [(8, 2, 1024, 128), (8, 4, 768, 96), (6, 2, 512, 64), (32, 8, 2048, 128)])
def test_single_segment_bitwise_equals_causal_grouped(H, Hkv, N, D):
    """Grouped-query heads: a single-segment packed call gives the causal
    call's bits too.  Group sizes 4 and 2 take the two-team dK/dV kernel in
    both calls (dense ones with mirrored key blocks at one round), the group
    of 3 the one-team kernel."""
    w = workloads.get("gqa_8k").with_(H=H, hkv=Hkv, N=N, D=D)
    say(f"B1 H{H} Hkv{Hkv} N{N} D{D} bf16 as one segment and as plain causal")
    t = w.tensors()
    seg = np.zeros((w.B, w.N), dtype=np.int32)
    packed = run_gpu(t, seg, w.dtype, w.scale, True)
    causal = run_gpu(t, None, w.dtype, w.scale, True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((packed[n] == causal[n]).all()), f"{n}: single-segment packed != causal"


def test_packed_long_documents_64k():
    w = workloads.get("packed_long_64k")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    seg = w.seg()
    out = run_gpu(t, seg, w.dtype, w.scale, True)
    lens = workloads.segment_lengths(seg[0])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    o_all, lse_all = down(out["o"]), down(out["lse"])
    rng = np.random.default_rng(5)
    # sampled rows of every head against the full-row oracle (explicit mask over all keys)
    for hh in range(w.H):
        rows = np.unique(np.concatenate([starts, starts + 1, rng.integers(0, w.N, 12), [w.N - 1]]))
        rows = rows[rows < w.N]
        o_r, l_r = attention_rows(t["q"][0, hh], t["k"][0, hh], t["v"][0, hh], rows, seg[0], w.scale, True)
        pv_r, _ = attention_rows(t["q"][0, hh], t["k"][0, hh], np.abs(t["v"][0, hh]), rows, seg[0], w.scale,
                                 True)
        check_o(o_all[0, hh, rows], o_r, w.dtype, f"O rows h{hh}", pv_r)
        check_lse(lse_all[0, hh, rows], l_r, w.dtype)
    # whole segments: a packed row equals each segment run alone
    order = np.argsort(lens)
    for si, hh in [(order[0], 0), (order[1], 7), (len(lens) - 1, 3)]:
        s0, L = int(starts[si]), int(lens[si])
        say(f"  oracle segment {si} [{s0}, {s0 + L}) head {hh}")
        tb = {n: t[n][:, hh:hh + 1, s0:s0 + L] for n in t}
        ref = _oracle_full(tb, None, w.scale, True)
        _compare(out, ref, w.dtype, (slice(0, 1), slice(hh, hh + 1), slice(s0, s0 + L)), f"[seg {si} h{hh}]")
    _invariants(out)


def test_packed_outputs_do_not_depend_on_other_segments():
    """Changing one segment's inputs leaves every other segment's results bit-identical."""
    import torch
    B, H, N, D = 1, 2, 1000, 128
    say("segment isolation B1 H2 N1000 D128")
    t = workloads.make_tensors(B, H, N, D, "bf16", 91)
    seg = workloads.random_segments(B, N, 91, max_len=300)
    a = run_gpu(t, seg, "bf16", 0.088, True)
    lens = workloads.segment_lengths(seg[0])
    s0, L = sum(lens[:1]), lens[1]
    t2 = {n: x.copy() for n, x in t.items()}
    for n in t2:
        t2[n][:, :, s0:s0 + L] = workloads.make_tensors(B, H, L, D, "bf16", 92)[n]
    b2 = run_gpu(t2, seg, "bf16", 0.088, True)
    keep = torch.ones(N, dtype=torch.bool, device="cuda")
    keep[s0:s0 + L] = False
    for n in ("o", "lse", "dq", "dk", "dv"):
        x, y = a[n][:, :, keep], b2[n][:, :, keep]
        assert bool((x == y).all()), f"{n} of other segments changed"


def test_grouped_query_heads_8k():
    """The pages' flagship attention shape: B1, 32 query / 8 key-value heads,
    N = 8192, D = 128, causal."""
    w = workloads.get("gqa_8k")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    out = run_gpu(t, None, w.dtype, w.scale, True)
    G = w.H // w.Hkv
    g = 5
    say(f"  oracle key/value head {g} with its {G} query heads")
    tb = {n: (t[n][:, g:g + 1] if n in ("k", "v") else t[n][:, g * G:(g + 1) * G]) for n in t}
    ref = _oracle_full(tb, None, w.scale, True)
    o, lse = down(out["o"][:, g * G:(g + 1) * G]), down(out["lse"][:, g * G:(g + 1) * G])
    check_o(o, ref["o"], w.dtype, pv_abs=ref["pv"])
    check_lse(lse, ref["lse"], w.dtype)
    check_grad(down(out["dq"][:, g * G:(g + 1) * G]), ref["dq"], w.dtype, "dq")
    check_grad(down(out["dk"][:, g:g + 1]), ref["dk"], w.dtype, "dk")
    check_grad(down(out["dv"][:, g:g + 1]), ref["dv"], w.dtype, "dv")
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.N - 1], rng.integers(0, w.N, 11)]))
    o_all, lse_all = down(out["o"]), down(out["lse"])
    for hh in range(w.H):
        o_r, l_r = attention_rows(t["q"][0, hh], t["k"][0, hh // G], t["v"][0, hh // G], rows, None,
                                  w.scale, True)
        pv_r, _ = attention_rows(t["q"][0, hh], t["k"][0, hh // G], np.abs(t["v"][0, hh // G]), rows, None,
                                 w.scale, True)
        check_o(o_all[0, hh, rows], o_r, w.dtype, f"O rows h{hh}", pv_r)
        check_lse(lse_all[0, hh, rows], l_r, w.dtype)
    _invariants(out)
    # the dK/dV teams add their halves of each group in a fixed order
    again = run_gpu(t, None, w.dtype, w.scale, True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((out[n] == again[n]).all()), f"{n} differs between identical runs"


def test_maximum_sequence_length():
    """The largest N the library accepts (FA_MAX_N = 2^22 tokens, one head,
    D = 64: 512 MiB per tensor), packed as 1024 documents of 4096 tokens so
    that the run stays short while every index, table and work list runs at
    full size.  The first, a middle and the last document are each checked
    against the oracle on that document alone (a packed row is each segment
    on its own)."""
    N, D, L = 1 << 22, 64, 4096
    say(f"maximum length B1 H1 N{N} D{D} bf16, {N // L} documents of {L}")
    t = workloads.make_tensors(1, 1, N, D, "bf16", 91)
    seg = np.repeat(np.arange(N // L, dtype=np.int32), L)[None]
    out = run_gpu(t, seg, "bf16", 0.125, True)
    for d in (0, N // L // 2, N // L - 1):
        r0, r1 = d * L, (d + 1) * L
        say(f"  document {d}: rows {r0}..{r1 - 1}")
        tb = {n: t[n][:, :, r0:r1] for n in t}
        ref = _oracle_full(tb, None, 0.125, True)
        check_o(down(out["o"][:, :, r0:r1]), ref["o"], "bf16", pv_abs=ref["pv"])
        check_lse(down(out["lse"][:, :, r0:r1]), ref["lse"], "bf16")
        for n in ("dq", "dk", "dv"):
            check_grad(down(out[n][:, :, r0:r1]), ref[n], "bf16", f"{n} document {d}")


def test_head_dim_96_8k():
    """head_dim 96 at a full-size causal shape: one whole head against the
    oracle, sampled rows of every head, and the identities."""
    w = workloads.get("causal_8k_d96")
    say(f"workload {w.name}: {w.note}")
    t = w.tensors()
    out = run_gpu(t, None, w.dtype, w.scale, True)
    b, h = 0, 11
    say(f"  oracle head b{b} h{h}")
    tb = {n: t[n][b:b + 1, h:h + 1] for n in t}
    _compare(out, _oracle_full(tb, None, w.scale, True), w.dtype, (slice(b, b + 1), slice(h, h + 1)),
             f"[b{b} h{h}]")
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.N - 1], rng.integers(0, w.N, 11)]))
    o_all, lse_all = down(out["o"]), down(out["lse"])
    for hh in range(w.H):
        o_r, l_r = attention_rows(t["q"][0, hh], t["k"][0, hh], t["v"][0, hh], rows, None, w.scale, True)
        pv_r, _ = attention_rows(t["q"][0, hh], t["k"][0, hh], np.abs(t["v"][0, hh]), rows, None, w.scale, True)
        check_o(o_all[0, hh, rows], o_r, w.dtype, f"O rows h{hh}", pv_r)
        check_lse(lse_all[0, hh, rows], l_r, w.dtype)
    _invariants(out)


def test_decreasing_segment_ids_are_flagged():
    """Segment ids must be non-decreasing along a row.  A row that breaks this
    gets unspecified values, but every access stays in bounds (shown for the
    schedule's index arithmetic by tests/test_schedule_model.py), the other
    rows are untouched, and the device sets workspace word 0, which the
    binding's check_seg turns into FaError (FA_ERR_SEG).  Valid ids leave the
    word at 0."""
    import torch
    import memory_efficient_attention_amd as fa
    B, H, N, D = 2, 2, 300, 64
    scale = 0.125
    say(f"decreasing segment ids B{B} H{H} N{N} D{D} bf16: row 1 bad, row 0 valid")
    t = workloads.make_tensors(B, H, N, D, "bf16", 93)
    good = workloads.random_segments(B, N, 93, max_len=70)
    bad = good.copy()
    bad[1] = bad[1][::-1].copy()                       # row 1: ids decrease
    assert fa.fa_check_seg(good) is None
    with pytest.raises(fa.FaError):
        fa.fa_check_seg(bad)
    q, k, v, do = (upload(t[n], "bf16") for n in ("q", "k", "v", "do"))
    dev = q.device
    ws_f = torch.zeros(fa.fa_workspace_bytes(B, H, N, D, True, False), dtype=torch.uint8, device=dev)
    ws_b = torch.zeros(fa.fa_workspace_bytes(B, H, N, D, True, True), dtype=torch.uint8, device=dev)

    def flag(ws):
        torch.cuda.synchronize()
        return int(ws[:4].view(torch.int32).item())

    for seg, want in ((bad, 1), (good, 0)):
        sg = upload_seg(seg)
        o, lse = fa.fa_fwd(q, k, v, sg, scale, True, workspace=ws_f)
        assert flag(ws_f) == want, f"forward flag {flag(ws_f)}, expected {want}"
        dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, sg, scale, True, workspace=ws_b)
        assert flag(ws_b) == want, f"backward flag {flag(ws_b)}, expected {want}"
        # row 0 is valid either way and must match the oracle
        t0 = {n: x[0:1] for n, x in t.items()}
        ref = _oracle_full(t0, seg[0:1], scale, True)
        out = dict(q=q[0:1], k=k[0:1], v=v[0:1], do=do[0:1], o=o[0:1], lse=lse[0:1], dq=dq[0:1],
                   dk=dk[0:1], dv=dv[0:1], seg=sg[0:1], scale=scale)
        _compare(out, ref, "bf16", tag=f"[row 0, row 1 {'bad' if want else 'valid'}]")
        if want:
            with pytest.raises(fa.FaError) as e:
                fa.fa_fwd(q, k, v, sg, scale, True, workspace=ws_f, check_seg=True)
            assert e.value.status == fa.FA_ERR_SEG
            with pytest.raises(fa.FaError) as e:
                fa.fa_bwd(q, k, v, o, do, lse, sg, scale, True, workspace=ws_b, check_seg=True)
            assert e.value.status == fa.FA_ERR_SEG
        else:
            fa.fa_fwd(q, k, v, sg, scale, True, workspace=ws_f, check_seg=True)
            fa.fa_bwd(q, k, v, o, do, lse, sg, scale, True, workspace=ws_b, check_seg=True)
