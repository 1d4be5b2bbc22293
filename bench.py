#!/usr/bin/env python3
"""Benchmark of the attention hot path: one step = fa_fwd + fa_bwd over one batch.

Prints ONE JSON line: effective TFLOP/s of forward + backward counting only
visible (unmasked) flops, 14 * D * V for V visible (query, key) pairs (4DV in
the forward's two products, 10DV in the backward's five), and its share of the
MI355X dense bf16 MFMA peak (2.5 PFLOP/s).  Inputs are seeded synthetic
tensors already resident in HBM when the timed region starts.

Beside the headline number the line carries
* ``roofline``: the dominant kernel's algorithmic flops per launch over its
  average launch time, measured with HIP events recorded on the launch stream
  around that kernel in a second pass of the same steps (the step time itself
  is taken with events at step boundaries only); ``traffic`` is its HBM bytes per
  launch from rocprofv3 counters (profiles/traffic.json), or null when the
  kernel sources changed since the counters were taken;
* ``cpu_baseline``: the fp64 oracle timed on this host on a bounded sample of
  the same workload (about 10 s of row blocks, see cpu_baseline).

Other modes: ``--all`` prints a table over every workload (and the causal
comparator of each packed one); ``--copy-calibration`` runs a plain
elementwise copy of known size (the reference for HBM byte counters);
``--ingest-counters`` turns rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
script into profiles/traffic.json.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s fwd+bwd (visible FLOPs) and % bf16 MFMA peak, N=8k/16k d=128"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "causal_16k"
KERNELS = ("fwd", "dq", "dkdv")     # in launch order; dQ also computes the per-row D_i
KERNEL_NAMES = {"fwd": "fwd_kernel", "dq": "dq_kernel", "dkdv": "dkdv_kernel"}


# ---------------------------------------------------------------- helpers

def visible_pairs(B, H, N, seg, causal=True) -> int:
    """Visible (query, key) pairs over all (batch, head): sum of L(L+1)/2 per segment."""
    import workloads
    per_row = []
    for b in range(B):
        lens = [N] if seg is None else workloads.segment_lengths(seg[b])
        per_row.append(sum(L * (L + 1) // 2 if causal else L * L for L in lens))
    return H * sum(per_row)


def kernel_sources_sha() -> str:
    """Hash of the sources the attention kernels (forward, dQ, dK/dV) are
    compiled from; the schedule, the loss layer and the host-side API files
    do not change them."""
    d = os.path.join(ROOT, "memory_efficient_attention_amd", "csrc")
    h = hashlib.sha256()
    for name in ("fa_bwd.hip", "fa_device.h", "fa_fwd.hip", "fa_internal.h"):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        import torch
        self.hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        vp = ctypes.c_void_p
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        self.hip.hipEventRecord.argtypes = [vp, vp]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.hip.hipEventDestroy.argtypes = [vp]
        self.made = []

    def new(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.made.append(e.value)
        return e.value

    def record(self, e: int, stream: int) -> None:
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


def alg_flops(kernel: str, D: int, V: int) -> float:
    """Credited (algorithmic) flops of one launch of each kernel, per visible
    pair: the step's 14 D is split as the forward's 4 D (S, P V), dQ's 6 D
    (the backward's one S recompute, dP, dQ) and dK/dV's 4 D (dV, dK).  The
    second S and dP that dK/dV recomputes are the split design's own cost and
    are not credited."""
    return {"fwd": 4.0, "dkdv": 4.0, "dq": 6.0}[kernel] * D * V


def executed_flops(kernel: str, D: int, V: int) -> float:
    """MFMA flops each kernel executes per visible pair (dK/dV computes S,
    dP, dV and dK: 8 D), for the matrix-unit utilisation next to the credit."""
    return {"fwd": 4.0, "dkdv": 8.0, "dq": 6.0}[kernel] * D * V


# ---------------------------------------------------------------- one workload

def alg_bytes(w) -> float:
    """Compulsory HBM bytes of one fwd + bwd step through the ABI: the
    forward reads q, k, v and writes o, lse; the backward reads q, k, v, o,
    dO, lse and writes dq, dk, dv.  Each (B, H, N, D) tensor once per use,
    k and v with their Hkv heads."""
    elt = 2 if w.dtype == "bf16" else 4
    tq = w.B * w.H * w.N * w.D * elt
    tkv = w.B * w.Hkv * w.N * w.D * elt
    return 6.0 * tq + 6.0 * tkv + 2.0 * w.B * w.H * w.N * 4


def run_workload(w, steps: int, warmup: int, seg_override="keep", causal=True, quiet=False, cold=False):
    """Time `steps` fwd+bwd steps after `warmup`.  cold: a 512 MiB scratch
    buffer is written between steps (outside the timed events), so no step
    finds its inputs in the 256 MB Infinity Cache; the step time is then the
    mean of the per-step event spans."""
    import numpy as np
    import torch

    import memory_efficient_attention_amd as fa

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t_np = w.tensors()
    x = {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in t_np.items()}
    seg_np = w.seg() if seg_override == "keep" else seg_override
    seg = None if seg_np is None else torch.from_numpy(seg_np).to(dev)
    B, H, N, D = w.B, w.H, w.N, w.D
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    ws_f = torch.empty(max(fa.fa_workspace_bytes(B, H, N, D, seg is not None, False), 256),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fa.fa_workspace_bytes(B, H, N, D, seg is not None, True), dtype=torch.uint8,
                       device=dev)
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def step(evs=None):
        if evs:
            ev.record(evs[0], stream)
        fa.fa_fwd(x["q"], x["k"], x["v"], seg, w.scale, causal, out=o, lse=lse, workspace=ws_f)
        if evs:
            ev.record(evs[1], stream)
        fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, seg, w.scale, causal, dq=dq, dk=dk, dv=dv,
                  workspace=ws_b, events=evs[2:5] if evs else None)

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None
    for _ in range(warmup):
        step()
    # Timed region 1, the step time: one event at each step boundary and none
    # inside a step (an event between two kernels drains the queue, which
    # costs the short workloads up to 0.1 ms a step).  Cold: the scratch
    # write sits outside the step's events.
    bounds = [[ev.new(), ev.new()] if cold else [ev.new()] for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev.record(bounds[0][-1], stream)
    for i in range(steps):
        if cold:
            scratch.fill_(i & 255)
            ev.record(bounds[i][-1], stream)
        step()
        ev.record(bounds[i + 1][0], stream)
    torch.cuda.synchronize()
    per_step = sorted(ev.ms(bounds[i][-1], bounds[i + 1][0]) for i in range(steps))
    total_ms = sum(per_step) if cold else ev.ms(bounds[0][-1], bounds[steps][0])
    # Timed region 2, the kernels: the same steps with events around each
    # kernel, for the per-kernel averages (the roofline's launch durations).
    stage_ev = [[ev.new() for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if cold:
            scratch.fill_(i & 255)
        step(stage_ev[i])
    torch.cuda.synchronize()
    stage = {k: 0.0 for k in KERNELS}
    for e in stage_ev:
        stage["fwd"] += ev.ms(e[0], e[1])
        stage["dq"] += ev.ms(e[2], e[3])
        stage["dkdv"] += ev.ms(e[3], e[4])
    stage = {k: v / steps for k, v in stage.items()}
    ev.close()
    ms = total_ms / steps
    V = visible_pairs(B, H, N, seg_np, causal)
    flops = 14.0 * D * V
    res = dict(ms=ms, V=V, flops=flops, tflops=flops / (ms * 1e-3) / 1e12, stage_ms=stage,
               ms_median=per_step[len(per_step) // 2], ms_min=per_step[0], t_np=t_np, seg_np=seg_np)
    del x, o, lse, dq, dk, dv, ws_f, ws_b, scratch
    torch.cuda.empty_cache()
    return res


CPU_BLOCK_ROWS = 1024
CPU_TARGET_SECONDS = 10.0


def cpu_baseline(w, t_np, seg_np, causal=True):
    """The fp64 oracle on a bounded sample of the workload, on this host's cores.

    The sample is made of blocks of CPU_BLOCK_ROWS query rows, taken from the
    end of (batch 0, head 0) backwards, then head 1, ..., until about
    CPU_TARGET_SECONDS of oracle work: per block the forward (O, LSE of those
    rows) and the backward (their dQ and their dK, dV contributions), each with
    the explicit mask over all N keys.  Credited flops are 14 * D times the
    visible pairs of the rows done."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention_backward_rows, attention_rows, visible_mask
    affinity = len(os.sched_getaffinity(0))
    threads = oracle_threads()
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        r = _cpu_sample(w, t_np, seg_np, causal, attention_rows, attention_backward_rows, visible_mask)
    r["cores"] = int(used)
    r["affinity_cores"] = affinity
    r["blas_env"] = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    r["sample"] += f"; cores = BLAS threads in use ({used}, set explicitly) of {affinity} in this process's affinity"
    return r


def oracle_threads() -> int:
    """BLAS threads for the oracle: OMP_NUM_THREADS when set (main() sets it,
    and OPENBLAS_NUM_THREADS, to the affinity count when absent), capped at
    the cores this process may run on."""
    affinity = len(os.sched_getaffinity(0))
    try:
        return max(1, min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity))))
    except ValueError:
        return affinity


def _cpu_sample(w, t_np, seg_np, causal, attention_rows, attention_backward_rows, visible_mask):
    import numpy as np
    b = 0
    seg_row = None if seg_np is None else seg_np[b]
    V, nrows, heads, el = 0, 0, set(), 0.0
    t0 = time.perf_counter()
    G = w.H // w.Hkv
    for h in range(w.H):
        s = {n: a[b, h // G if n in ("k", "v") else h] for n, a in t_np.items()}
        for hi in range(w.N, 0, -CPU_BLOCK_ROWS):
            rows = np.arange(max(0, hi - CPU_BLOCK_ROWS), hi)
            o_r, lse_r = attention_rows(s["q"], s["k"], s["v"], rows, seg_row, w.scale, causal)
            attention_backward_rows(s["q"], s["k"], s["v"], s["do"], o_r, lse_r, rows, seg_row,
                                    w.scale, causal)
            V += int(visible_mask(rows, w.N, seg_row, causal).sum())
            nrows += rows.size
            heads.add(h)
            el = time.perf_counter() - t0
            if el >= CPU_TARGET_SECONDS:
                break
        if el >= CPU_TARGET_SECONDS:
            break
    return {"value": round(14.0 * w.D * V / el / 1e12, 6), "unit": "TFLOP/s", "cores": 0,
            "kind": "oracle",
            "sample": f"{nrows} query rows of batch 0 over {len(heads)} head(s), last rows first, of "
                      f"N={w.N}, D={w.D}: fp64 forward + backward with the explicit mask over all keys "
                      f"({V} visible pairs, {el:.1f} s)",
            "seconds": round(el, 2)}


def roofline(w, res):
    stage = res["stage_ms"]
    dom = max(("fwd", "dkdv", "dq"), key=lambda k: stage[k])
    avg_ms = stage[dom]
    alg = alg_flops(dom, w.D, res["V"])
    achieved = alg / (avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    traffic = None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(path):
        try:
            with open(path) as f:
                rec = json.load(f).get(w.name, {}).get(dom)
            if rec and rec.get("source_sha") == kernel_sources_sha():
                traffic = rec["bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            traffic = None
    executed = executed_flops(dom, w.D, res["V"]) / (avg_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": KERNEL_NAMES[dom],
            "avg_ms": round(avg_ms, 4), "alg_flops_per_launch": alg,
            "executed_flops_per_launch": executed_flops(dom, w.D, res["V"]),
            "executed_tflops": round(executed, 2), "executed_frac": round(executed / peak, 4),
            "per_kernel_frac": {k: round(alg_flops(k, w.D, res["V"]) / (stage[k] * 1e-3) / 1e12 / peak, 4)
                                for k in ("fwd", "dkdv", "dq")}}


# ---------------------------------------------------------------- modes

def eight_k(steps, warmup):
    """The 8k half of the metric: causal N=8192 D=128 (B1 H32 bf16) and the
    same inputs through the packed path as one segment (identical work), with
    the packed path's overhead over causal."""
    import workloads
    w = workloads.get("single_segment_8k")
    c = run_workload(w, steps, warmup, seg_override=None)
    p = run_workload(w, steps, warmup)
    assert c["V"] == p["V"]
    row = lambda r: {"ms_per_step": round(r["ms"], 4), "step_ms_median": round(r["ms_median"], 4),
                     "tflops": round(r["tflops"], 2),
                     "pct_bf16_peak": round(100.0 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
                     "stages_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()}}
    return {"workload": "B1 H32 N8192 D128 bf16, causal; and the same inputs as one segment through the "
                        "packed path", "visible_pairs": c["V"], "causal": row(c), "packed_one_segment": row(p),
            "packed_overhead_vs_causal": round(p["ms"] / c["ms"] - 1.0, 4)}


def headline(args):
    import workloads
    w = workloads.get(args.workload)
    res = run_workload(w, args.steps, args.warmup)
    out = {
        "metric": METRIC,
        "value": round(res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        "step_ms_median": round(res["ms_median"], 4),
        "step_ms_min": round(res["ms_min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q, k, v, dO)",
        "config": {"workload": f"{w.name}: {w.note}", "global_batch": w.B, "seq_len": w.N,
                   "heads": w.H, "kv_heads": w.Hkv, "head_dim": w.D, "causal": True,
                   "segments": "none" if w.layout == "none" else w.layout,
                   "visible_pairs": res["V"], "visible_flops": res["flops"]},
        "pct_bf16_peak": round(100.0 * res["tflops"] / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {k: round(v, 4) for k, v in res["stage_ms"].items()},
        "roofline": roofline(w, res),
        "n8k": eight_k(args.steps, args.warmup) if w.name == DEFAULT_WORKLOAD and not args.no_8k else None,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, res["t_np"], res["seg_np"])
    print(json.dumps(out), flush=True)


def run_lce(steps, warmup):
    """Time the fused linear cross-entropy at the pages' loss-layer shape
    (N = 8192, V = 151936, D = 4096, bf16): fa_lce_fwd, then fa_lce_bwd with
    dh and dW, each bracketed by HIP events on the current stream."""
    import torch
    import workloads
    import memory_efficient_attention_amd as fa
    c = workloads.LCE_WORKLOAD
    N, V, D = c["N"], c["V"], c["D"]
    print(f"# generating {c['name']} inputs", file=sys.stderr, flush=True)
    x = workloads.make_lce_inputs(N, V, D, c["seed"])
    h = torch.from_numpy(x["h"]).cuda().to(torch.bfloat16)
    w = torch.from_numpy(x["w"]).cuda().to(torch.bfloat16)
    del x["w"]
    t = torch.from_numpy(x["targets"]).cuda()
    g = torch.from_numpy(x["dnll"]).cuda()
    ws_f = torch.empty(fa.fa_lce_workspace_bytes(N, V, D, False), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(fa.fa_lce_workspace_bytes(N, V, D, True), dtype=torch.uint8, device="cuda")
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    lse = None
    for _ in range(warmup):
        _, lse, _ = fa.fa_lce_fwd(h, w, t, workspace=ws_f)
        fa.fa_lce_bwd(h, w, t, lse, g, workspace=ws_b)
    E = [[ev.new() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in E:
        ev.record(e[0], stream)
        _, lse, _ = fa.fa_lce_fwd(h, w, t, workspace=ws_f)
        ev.record(e[1], stream)
        fa.fa_lce_bwd(h, w, t, lse, g, workspace=ws_b)
        ev.record(e[2], stream)
    torch.cuda.synchronize()
    fwd = sum(ev.ms(e[0], e[1]) for e in E) / steps
    bwd = sum(ev.ms(e[1], e[2]) for e in E) / steps
    ev.close()
    flop = 2.0 * N * V * D
    return {"workload": c["name"], "fwd_ms": round(fwd, 3), "bwd_ms": round(bwd, 3),
            "fwd_tflops": round(flop / (fwd * 1e-3) / 1e12, 1),
            # backward: logits recomputed, dh = dZ W, dW = dZ^T H
            "bwd_tflops": round(3 * flop / (bwd * 1e-3) / 1e12, 1),
            "workspace_bytes": {"fwd": ws_f.numel(), "bwd": ws_b.numel()},
            "logits_bytes_bf16": N * V * 2}


def report_all(args):
    import workloads
    rows = []
    names = ["tiny_causal_fp32", "causal_2k", "packed_short_4k", "single_segment_8k", "causal_16k",
             "packed_long_64k", "gqa_8k", "causal_8k_d96"]
    for name in names:
        w = workloads.get(name)
        print(f"# running {name}", file=sys.stderr, flush=True)
        r = run_workload(w, args.steps, args.warmup)
        row = dict(workload=name, ms=r["ms"], ms_median=r["ms_median"], ms_min=r["ms_min"],
                   tflops=r["tflops"], V=r["V"], stages=r["stage_ms"],
                   alg_gbs=alg_bytes(w) / (r["ms"] * 1e-3) / 1e9)
        if w.layout in ("short", "long", "single"):
            c = run_workload(w, args.steps, args.warmup, seg_override=None)
            row["causal_ms"] = c["ms"]
            row["causal_V"] = c["V"]
            row["speedup_vs_causal"] = c["ms"] / r["ms"]
            row["visible_ratio"] = c["V"] / r["V"]
        if w.layout == "short":
            # short examples fit the Infinity Cache; time them cold as well
            k = run_workload(w, args.steps, args.warmup, cold=True)
            row["cold_ms"] = k["ms"]
            row["cold_ms_median"] = k["ms_median"]
        rows.append(row)
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()}),
              flush=True)
    print("\n| workload | ms fwd+bwd (mean) | median | min | fwd | dQ (with D_i) | dK/dV | eff. TFLOP/s | % peak | "
          "algorithmic GB/s | packed speedup vs causal (visible ratio) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        s = r["stages"]
        sp = (f"{r['speedup_vs_causal']:.2f}x ({r['visible_ratio']:.2f}x) against causal {r['causal_ms']:.3f} ms "
              f"({14 * r['causal_V'] * workloads.get(r['workload']).D / (r['causal_ms'] * 1e-3) / 1e12:.0f} TFLOP/s)"
              if "speedup_vs_causal" in r else "")
        if "cold_ms" in r:
            sp += f"; cache-cold {r['cold_ms']:.3f} ms"
        print(f"| {r['workload']} | {r['ms']:.3f} | {r['ms_median']:.3f} | {r['ms_min']:.3f} | {s['fwd']:.3f} | "
              f"{s['dq']:.3f} | {s['dkdv']:.3f} | {r['tflops']:.1f} | "
              f"{100 * r['tflops'] / PEAK_BF16_TFLOPS:.1f} | {r['alg_gbs']:.0f} | {sp} |")


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain copy of COPY_BYTES (read once, written once): torch.neg into a
    second buffer, timed by the counters, not by us."""
    import torch
    n = COPY_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "kernel": "neg"}), flush=True)


def _counter_rows(path):
    """(kernel name, counter name, value) rows of rocprofv3 counter CSVs under path."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""),
                             float(r.get("Counter_Value", "nan"))))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {path}")
    return rows


def _avg(rows, counter, match):
    vals = [v for k, c, v in rows if c == counter and match in k]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {match!r}")
    return sum(vals) / len(vals), len(vals)


def ingest_counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, workload):
    """profiles/traffic.json entry: HBM bytes per launch of each attention
    kernel = counter (KiB per dispatch) scaled so that the plain copy reads
    and writes exactly COPY_BYTES."""
    f_rows, w_rows = _counter_rows(fetch_dir), _counter_rows(write_dir)
    cf, _ = _avg(_counter_rows(cal_fetch_dir), "FETCH_SIZE", "neg")
    cw, _ = _avg(_counter_rows(cal_write_dir), "WRITE_SIZE", "neg")
    kf, kw = COPY_BYTES / cf, COPY_BYTES / cw          # bytes per counter unit
    entry = {}
    for short, name in KERNEL_NAMES.items():
        try:
            fv, n = _avg(f_rows, "FETCH_SIZE", name)
            wv, _ = _avg(w_rows, "WRITE_SIZE", name)
        except SystemExit:
            continue
        entry[short] = {"kernel": name, "dispatches": n, "fetch_bytes": fv * kf, "write_bytes": wv * kw,
                        "bytes_per_launch": fv * kf + wv * kw, "source_sha": kernel_sources_sha()}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[workload] = entry
    data["_calibration"] = {"copy_bytes": COPY_BYTES, "fetch_counter_per_copy": cf,
                            "write_counter_per_copy": cw, "bytes_per_fetch_unit": kf,
                            "bytes_per_write_unit": kw}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


def summarize_trace(path, warmup):
    """Per-kernel launch statistics from a rocprofv3 --kernel-trace run of
    this script, one row per (kernel, grid size) so that the headline
    workload and the 8k ones stay apart: the first `warmup` dispatches of
    each row (the untimed warm-up steps) are dropped, the rest summarised
    (ms)."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {path}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "")
                if not any(n in name for n in KERNEL_NAMES.values()):
                    continue
                grid = r.get("Grid_Size_X") or r.get("Grid_Size") or "?"
                wg = r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or "?"
                per.setdefault((name, grid, wg), []).append(
                    (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6))
    out = []
    for (name, grid, wg), v in sorted(per.items(), key=lambda kv: min(t for t, _ in kv[1])):
        d = [x for _, x in sorted(v)][warmup:]
        if not d:
            continue
        out.append({"kernel": name, "grid_threads": grid, "workgroup": wg, "calls": len(d),
                    "avg_ms": round(statistics.fmean(d), 4), "median_ms": round(statistics.median(d), 4),
                    "min_ms": round(min(d), 4), "max_ms": round(max(d), 4)})
    print(json.dumps(out, indent=1))


def summarize_counters(path):
    """Per (kernel, grid size) averages of every counter in the rocprofv3
    --pmc runs under path (all dispatches)."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "")
                if not any(n in name for n in KERNEL_NAMES.values()):
                    continue
                key = (name, r.get("Grid_Size") or r.get("Grid_Size_X") or "?")
                d = acc.setdefault(key, {})
                d.setdefault((r.get("Dispatch_Id"), r["Counter_Name"]), 0.0)
                d[(r.get("Dispatch_Id"), r["Counter_Name"])] += float(r["Counter_Value"])
    out = []
    for (name, grid), d in sorted(acc.items()):
        per = {}
        for (disp, cname), v in d.items():
            per.setdefault(cname, []).append(v)
        out.append({"kernel": name, "grid_threads": grid,
                    "dispatches": max(len(v) for v in per.values()),
                    "avg": {c: sum(v) / len(v) for c, v in sorted(per.items())}})
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-8k", action="store_true", help="leave out the 8k fields (profiling runs of one shape)")
    ap.add_argument("--all", action="store_true", help="table over every workload instead of the JSON line")
    ap.add_argument("--lce", action="store_true", help="time the fused linear cross-entropy loss layer")
    ap.add_argument("--copy-calibration", action="store_true", help="plain copy of known size for counters")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR",
                                                           "CAL_WRITE_DIR"),
                    help="write profiles/traffic.json from rocprofv3 counter runs (CPU only)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="per-kernel statistics of a rocprofv3 kernel trace of this script, warm-up dropped")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="per-kernel averages of the counters of a rocprofv3 --pmc run of this script")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.warmup)
        return
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, args.workload)
        return
    # the oracle's BLAS threads, set before numpy (through torch) loads them
    ncpu = str(len(os.sched_getaffinity(0)))
    os.environ.setdefault("OMP_NUM_THREADS", ncpu)
    os.environ.setdefault("OPENBLAS_NUM_THREADS", os.environ["OMP_NUM_THREADS"])
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this attention path runs on one GPU (one process, one device); runs on more "
              "than one GPU are not part of it.  It would shard across GPUs by batch and head, with "
              "no exchange between them.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
    elif args.lce:
        print(json.dumps(run_lce(args.steps, args.warmup)), flush=True)
    elif args.all:
        report_all(args)
    else:
        headline(args)


if __name__ == "__main__":
    main()
