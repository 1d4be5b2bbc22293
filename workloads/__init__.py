"""Seeded synthetic inputs for the attention workloads.

This module only draws numbers: segment layouts (per-token segment ids) and the
Q, K, V, dO tensors.  It holds none of the attention arithmetic, so both the
fp64 oracle and the HIP path can take their inputs from here without sharing
any computation.

Every draw uses numpy's PCG64 ``default_rng``: layouts come from
``default_rng([seed, 0])`` and tensors from ``default_rng([seed, 1])``.  Q, K, V
and dO are drawn in that order as float32 N(0, 1) of shape (B, H, N, D) and,
for bf16 workloads, rounded to bf16 (round to nearest, ties to even).  The
float32 arrays returned are exactly the values the GPU receives.

The packed layouts stand in for the datasets the pages measure on (an
instruction-tuning set of short examples packed into 4,096-token rows, and long
documents); no item of any dataset is reproduced, only the length statistics.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "bf16_bits", "bf16_round",
    "make_tensors", "seg_from_lengths", "segment_lengths",
    "layout_short_examples", "layout_long_documents", "random_segments",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value, returned as float32.

    The same rounding as bf16_bits, done in 32-bit integers: adding at most
    0x8000 cannot wrap for any finite value or infinity (only NaN patterns sit
    that close to 2^32), so no 64-bit temporaries are needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = (bf16_bits(x[nan]).astype(np.uint32) << 16)
    return r.view(np.float32)


def seg_from_lengths(rows: list[list[int]], N: int) -> np.ndarray:
    """Per-token segment ids (B, N) int32 from per-row segment lengths.

    Ids start at 0 in every row and increase by one per segment, so each row is
    non-decreasing.  Each row's lengths must sum to N.
    """
    seg = np.empty((len(rows), N), dtype=np.int32)
    for b, lens in enumerate(rows):
        if sum(lens) != N or min(lens) < 1:
            raise ValueError(f"row {b}: lengths {lens} do not tile {N} tokens")
        seg[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    return seg


def segment_lengths(seg_row: np.ndarray) -> list[int]:
    """Lengths of the contiguous runs of equal ids in one row."""
    seg_row = np.asarray(seg_row)
    if seg_row.size == 0:
        return []
    cut = np.flatnonzero(np.diff(seg_row) != 0) + 1
    edges = np.concatenate([[0], cut, [seg_row.size]])
    return [int(e) for e in np.diff(edges)]


def layout_short_examples(B: int, N: int, seed: int, median: float = 84.0,
                          sigma: float = 0.8, lo: int = 8, hi: int = 1024) -> np.ndarray:
    """Rows packed first-fit with short examples, trailing pad as its own segment.

    Lengths are lognormal with the given median and sigma, rounded and clipped
    to [lo, hi], drawn until the pool holds 1.5 * B * N tokens.  The pool is
    shuffled with the same seeded generator, then each item goes into the first
    row with room for it; an item that fits nowhere is dropped.  What is left of
    a row becomes one pad segment with its own id.
    """
    rng = np.random.default_rng([seed, 0])
    pool: list[int] = []
    total = 0
    while total < 1.5 * B * N:
        n = int(np.clip(np.rint(rng.lognormal(math.log(median), sigma)), lo, hi))
        pool.append(n)
        total += n
    order = rng.permutation(len(pool))
    rows: list[list[int]] = [[] for _ in range(B)]
    room = [N] * B
    for idx in order:
        n = pool[idx]
        for b in range(B):
            if room[b] >= n:
                rows[b].append(n)
                room[b] -= n
                break
    for b in range(B):
        if room[b] > 0:
            rows[b].append(room[b])
    return seg_from_lengths(rows, N)


def layout_long_documents(B: int, N: int, seed: int, lo: int = 1024,
                          hi: int = 16384) -> np.ndarray:
    """Rows filled with documents of integer-uniform length in [lo, hi].

    Documents are drawn until the row is full; the last one is truncated.
    """
    rng = np.random.default_rng([seed, 0])
    rows = []
    for _ in range(B):
        lens, used = [], 0
        while used < N:
            n = int(rng.integers(lo, hi + 1))
            n = min(n, N - used)
            lens.append(n)
            used += n
        rows.append(lens)
    return seg_from_lengths(rows, N)


def random_segments(B: int, N: int, seed: int, max_len: int | None = None) -> np.ndarray:
    """Random contiguous segments (lengths uniform in [1, max_len]) for small tests."""
    rng = np.random.default_rng([seed, 2])
    max_len = max_len or max(1, N // 3)
    rows = []
    for _ in range(B):
        lens, used = [], 0
        while used < N:
            n = min(int(rng.integers(1, max_len + 1)), N - used)
            lens.append(n)
            used += n
        rows.append(lens)
    return seg_from_lengths(rows, N)


def make_tensors(B: int, H: int, N: int, D: int, dtype: str, seed: int,
                 names=("q", "k", "v", "do"), Hkv: int | None = None) -> dict[str, np.ndarray]:
    """Q and dO as float32 (B, H, N, D), K and V as (B, Hkv, N, D) (Hkv = H
    unless given), iid N(0, 1), bf16-rounded for bf16.

    The four tensors are always drawn in the order q, k, v, do from one
    generator, so asking for a subset still returns the same values.
    """
    rng = np.random.default_rng([seed, 1])
    Hkv = H if Hkv is None else Hkv
    out = {}
    for name in ("q", "k", "v", "do"):
        x = rng.standard_normal((B, Hkv if name in ("k", "v") else H, N, D), dtype=np.float32)
        if name not in names:
            continue
        if dtype == "bf16":
            x = bf16_round(x)
        elif dtype != "fp32":
            raise ValueError(f"dtype {dtype!r}")
        out[name] = x
    return out


@dataclass(frozen=True)
class Workload:
    """One synthetic attention workload: shapes, dtype, layout recipe, seed."""
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    layout: str          # "none" (plain causal), "single" (seg = 0), "short", "long"
    seed: int
    causal: bool = True
    hkv: int = 0         # key/value heads; 0 means H (no grouping)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def Hkv(self) -> int:
        return self.hkv or self.H

    def seg(self) -> np.ndarray | None:
        if self.layout == "none":
            return None
        if self.layout == "single":
            return np.zeros((self.B, self.N), dtype=np.int32)
        if self.layout == "short":
            return layout_short_examples(self.B, self.N, self.seed)
        if self.layout == "long":
            return layout_long_documents(self.B, self.N, self.seed)
        raise ValueError(self.layout)

    def tensors(self, names=("q", "k", "v", "do")) -> dict[str, np.ndarray]:
        return make_tensors(self.B, self.H, self.N, self.D, self.dtype, self.seed, names, self.Hkv)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny_causal_fp32": Workload("tiny_causal_fp32", 1, 2, 256, 64, "fp32", "single", 1,
                                 note="B1 H2 N256 D64 fp32, one segment (seg id 0)"),
    "causal_2k": Workload("causal_2k", 1, 32, 2048, 128, "bf16", "none", 2,
                          note="B1 H32 N2048 D128 bf16, causal"),
    "packed_short_4k": Workload("packed_short_4k", 4, 32, 4096, 128, "bf16", "short", 3,
                                note="B4 H32 N4096 D128 bf16, lognormal short examples"),
    "causal_16k": Workload("causal_16k", 1, 32, 16384, 128, "bf16", "none", 4,
                           note="B1 H32 N16384 D128 bf16, causal"),
    "single_segment_8k": Workload("single_segment_8k", 1, 32, 8192, 128, "bf16", "single", 4,
                                  note="B1 H32 N8192 D128 bf16, packed path with one segment"),
    "packed_long_64k": Workload("packed_long_64k", 1, 8, 65536, 64, "bf16", "long", 5,
                                note="B1 H8 N65536 D64 bf16, documents U[1024,16384]"),
    "gqa_8k": Workload("gqa_8k", 1, 32, 8192, 128, "bf16", "none", 6, hkv=8,
                       note="B1 H32 (8 KV heads) N8192 D128 bf16, causal"),
    "causal_8k_d96": Workload("causal_8k_d96", 1, 32, 8192, 96, "bf16", "none", 7,
                              note="B1 H32 N8192 D96 bf16, causal"),
}


def make_lce_inputs(N: int, V: int, D: int, seed: int, targets_edge: bool = False) -> dict[str, np.ndarray]:
    """Inputs of the linear cross-entropy loss layer: hidden states h (N, D)
    iid N(0, 1), a head w (V, D) iid N(0, 1/D) (so that logits are O(1), as
    after a normalised final layer), both bf16-rounded, targets (N,) int32
    uniform over [0, V), and per-token upstream gradients dnll (N,) = 1/N (a
    mean).  With targets_edge the first and last targets are 0 and V - 1."""
    rng = np.random.default_rng([seed, 3])
    h = bf16_round(rng.standard_normal((N, D), dtype=np.float32))
    w = np.empty((V, D), dtype=np.float32)
    for r0 in range(0, V, 8192):                  # bounded temporaries at V = 151936
        r1 = min(r0 + 8192, V)
        w[r0:r1] = bf16_round(rng.standard_normal((r1 - r0, D), dtype=np.float32) / np.float32(np.sqrt(D)))
    t = rng.integers(0, V, N).astype(np.int32)
    if targets_edge and N >= 2:
        t[0], t[-1] = 0, V - 1
    return {"h": h, "w": w, "targets": t, "dnll": np.full(N, 1.0 / N, dtype=np.float32)}


LCE_WORKLOAD = dict(name="lce_8k", N=8192, V=151936, D=4096, seed=8,
                    note="N8192 V151936 D4096 bf16 fused linear cross-entropy")


def get(name: str) -> Workload:
    return WORKLOADS[name]
