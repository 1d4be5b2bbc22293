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
