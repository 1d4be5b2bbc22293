"""Host-side checks of the benchmark's bookkeeping (no GPU): the visible-pair
count behind the effective-TFLOP/s metric, the per-kernel algorithmic work,
and the refusal of multi-GPU runs."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def _brute_pairs(B, H, N, seg, causal):
    """Count (query, key) pairs the mask lets through, one by one."""
    n = 0
    for b in range(B):
        for i in range(N):
            for j in range(N):
                if causal and j > i:
                    continue
                if seg is not None and seg[b, i] != seg[b, j]:
                    continue
                n += 1
    return H * n


def test_visible_pairs_matches_brute_force():
    for B, N, max_len in ((1, 1, 1), (2, 17, 5), (3, 64, 64), (2, 50, 1)):
        seg = workloads.random_segments(B, N, 31 + N, max_len=max_len)
        for causal in (True, False):
            assert bench.visible_pairs(B, 3, N, seg, causal) == _brute_pairs(B, 3, N, seg, causal)
        assert bench.visible_pairs(B, 2, N, None) == _brute_pairs(B, 2, N, None, True)


def test_visible_pairs_at_the_bench_shape():
    # causal N = 16384, 32 heads: 32 * N (N + 1) / 2
    assert bench.visible_pairs(1, 32, 16384, None) == 32 * 16384 * 16385 // 2 == 4295229440


def test_algorithmic_flops_per_kernel():
    D, V = 128, 1000
    # credited: the step's 14 D V split as forward 4, dQ 6 (one S recompute,
    # dP, dQ), dK/dV 4 (dV, dK)
    assert bench.alg_flops("fwd", D, V) == 4 * D * V
    assert bench.alg_flops("dkdv", D, V) == 4 * D * V
    assert bench.alg_flops("dq", D, V) == 6 * D * V
    assert sum(bench.alg_flops(k, D, V) for k in ("fwd", "dkdv", "dq")) == 14 * D * V
    # executed: dK/dV recomputes S and dP as well, 18 D V in all
    assert bench.executed_flops("dkdv", D, V) == 8 * D * V
    assert sum(bench.executed_flops(k, D, V) for k in ("fwd", "dkdv", "dq")) == 18 * D * V


def test_oracle_threads_follow_the_environment(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.oracle_threads() == 1
    monkeypatch.setenv("OMP_NUM_THREADS", str(n + 100))
    assert bench.oracle_threads() == n
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.oracle_threads() == n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_trace_summary_drops_warmup_per_kernel_and_grid(tmp_path, capsys):
    """--summarize-trace keeps the headline and 8k dispatches of one kernel
    apart by grid size and drops the first `warmup` of each."""
    import json
    rows = ["Kernel_Name,Grid_Size_X,Workgroup_Size_X,Start_Timestamp,End_Timestamp"]
    t = 0
    for grid, durs in (("1048576", [9, 9, 2, 2, 2]), ("524288", [7, 1, 1])):
        for d in durs:
            rows.append(f"fa::dkdv_kernel<x>,{grid},512,{t},{t + d * 1000000}")
            t += 10 ** 8
    (tmp_path / "a_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_trace(str(tmp_path), 2)
    out = json.loads(capsys.readouterr().out)
    by_grid = {r["grid_threads"]: r for r in out}
    assert by_grid["1048576"]["calls"] == 3 and by_grid["1048576"]["avg_ms"] == 2.0
    assert by_grid["524288"]["calls"] == 1 and by_grid["524288"]["avg_ms"] == 1.0


def test_counter_summary_averages_per_dispatch(tmp_path, capsys):
    """--summarize-counters sums a counter's instances within a dispatch,
    then averages over dispatches, per (kernel, grid)."""
    import json
    rows = ["Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value"]
    for disp, vals in ((1, (3, 5)), (2, (4, 4))):
        for v in vals:   # two instances (e.g. XCDs) of one counter per dispatch
            rows.append(f"{disp},fa::dq_kernel<x>,1024,SQ_INSTS_MFMA,{v}")
    rows.append("3,other_kernel,64,SQ_INSTS_MFMA,100")
    (tmp_path / "p_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_counters(str(tmp_path))
    out = json.loads(capsys.readouterr().out)
    assert len(out) == 1 and out[0]["dispatches"] == 2 and out[0]["avg"]["SQ_INSTS_MFMA"] == 8.0


def test_algorithmic_bytes_follow_the_abi():
    """Compulsory bytes of one fwd + bwd step: every tensor the two calls
    read or write, once per call that touches it (brute-force list)."""
    for name in ("causal_16k", "gqa_8k", "tiny_causal_fp32", "packed_short_4k"):
        w = workloads.get(name)
        elt = 2 if w.dtype == "bf16" else 4
        q = w.B * w.H * w.N * w.D * elt
        kv = w.B * w.Hkv * w.N * w.D * elt
        rows = w.B * w.H * w.N * 4
        fwd = [q, kv, kv, q, rows]                      # read q k v, write o lse
        bwd = [q, kv, kv, q, q, rows, q, kv, kv]        # read q k v o dO lse, write dq dk dv
        assert bench.alg_bytes(w) == sum(fwd) + sum(bwd)
    assert bench.alg_bytes(workloads.get("causal_16k")) == 1614807040
