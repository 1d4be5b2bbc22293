"""A host model of the segment schedule's index arithmetic (the table and
order kernels of the packed path), run on segment ids that DEcrease.

The library's contract for such ids is: values unspecified, every memory
access in bounds, and the workspace flag raised.  The kernels' only indices
that come from the ids are the per-tile ranges of the tables; everything else
(batch, tile, row) comes from the grid.  This model repeats the kernels'
integer steps (binary searches over the row, clamp, division by the tile) and
checks that, whatever the ids, every range names tiles inside the row, the
work list is a permutation of the (batch, tile) pairs, and a walk over an
inverted range (first > last) makes no iteration.  No GPU is used.
"""
import numpy as np
import pytest


def first_at_least(s, v):
    lo, hi = 0, len(s)
    while lo < hi:
        mid = (lo + hi) >> 1
        assert 0 <= mid < len(s)          # every probe reads inside the row
        if s[mid] < v:
            lo = mid + 1
        else:
            hi = mid
    return lo


def first_above(s, v):
    lo, hi = 0, len(s)
    while lo < hi:
        mid = (lo + hi) >> 1
        assert 0 <= mid < len(s)
        if s[mid] <= v:
            lo = mid + 1
        else:
            hi = mid
    return lo


def table(seg, tile, other, keys, causal):
    """Per-tile {first, last} ranges of one table job, as the table kernel
    computes them."""
    B, N = seg.shape
    nt = (N + tile - 1) // tile
    out = np.zeros((B, nt, 2), dtype=np.int64)
    for b in range(B):
        s = seg[b]
        for it in range(nt):
            r0, r1 = it * tile, min(it * tile + tile, N) - 1
            if keys:
                lo = r0 if causal else first_at_least(s, s[r0])
                hi = first_above(s, s[r1]) - 1
            else:
                lo = first_at_least(s, s[r0])
                hi = r1 if causal else first_above(s, s[r1]) - 1
            lo, hi = min(max(lo, 0), N - 1), min(max(hi, 0), N - 1)
            out[b, it] = (lo // other, hi // other)
    return out


def order(tab):
    """Longest-first work list {b, tile, first, last} by the order kernel's
    counting sort (256 buckets of clamped range length)."""
    B, nt, _ = tab.shape
    NB = 256
    flat = tab.reshape(-1, 2)
    bucket = NB - 1 - np.clip(flat[:, 1] - flat[:, 0] + 1, 0, NB - 1)
    cnt = np.bincount(bucket, minlength=NB)
    start = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    work = np.full((B * nt, 4), -1, dtype=np.int64)
    for i in range(B * nt):
        k = start[bucket[i]]
        start[bucket[i]] += 1
        assert 0 <= k < B * nt
        work[k] = (i // nt, i % nt, flat[i, 0], flat[i, 1])
    return work


def walk_trips(first, last, sub=1):
    """Iterations of a kernel's tile walk over [first, last] with `sub` tiles
    per ring slot (the kernels' (last - first + sub) / sub, C division)."""
    n = last - first + sub
    return int(n / sub) if n >= 0 else -int(-n / sub)


def _bad_rows(rng, B, N):
    """Rows of ids that decrease somewhere: reversed runs, a single dip, and
    random ids."""
    rows = []
    for kind in range(B):
        if kind % 3 == 0:
            lens = rng.integers(1, max(2, N // 3), size=N)
            ids = np.repeat(np.arange(len(lens))[::-1], lens)[:N]
        elif kind % 3 == 1:
            ids = np.repeat(np.arange(N // 4 + 1), 4)[:N].copy()
            ids[rng.integers(1, N) if N > 1 else 0] = -7
        else:
            ids = rng.integers(-50, 50, size=N)
        rows.append(ids.astype(np.int32))
    return np.stack(rows)


# the (tile, other) pairs the library uses: forward / dQ query tiles of
# 128 or 256 rows over 64-key tiles, dK/dV key tiles of 128 or 256 rows over
# 32-query tiles
JOBS = [(256, 64, 0), (128, 64, 0), (128, 32, 1), (256, 32, 1)]


@pytest.mark.parametrize("N", [1, 2, 31, 64, 255, 257, 1000])
@pytest.mark.parametrize("causal", [True, False])
def test_decreasing_ids_keep_every_range_in_bounds(N, causal):
    rng = np.random.default_rng(N + 17 * causal)
    seg = _bad_rows(rng, 6, N)
    for tile, other, keys in JOBS:
        tab = table(seg, tile, other, keys, causal)
        n_other = (N + other - 1) // other
        assert (tab >= 0).all() and (tab <= n_other - 1).all()
        work = order(tab)
        B, nt = tab.shape[:2]
        # a permutation of every (batch, tile) pair
        pairs = sorted(map(tuple, work[:, :2].tolist()))
        assert pairs == [(b, t) for b in range(B) for t in range(nt)]
        for b, t, lo, hi in work.tolist():
            for sub in (1, 2):
                trips = walk_trips(lo, hi, sub)
                if hi < lo:
                    assert trips <= 0          # the loop body never runs
                else:
                    # every tile the walk touches lies inside [lo, hi], so
                    # inside the row
                    touched = [lo + sub * j + i for j in range(trips) for i in range(sub)
                               if lo + sub * j + i <= hi]
                    assert touched == list(range(lo, hi + 1))


def test_valid_ids_give_the_exact_visible_ranges():
    """With non-decreasing ids the model's ranges cover exactly the tiles that
    hold a visible pair (checked by brute force), so the model is the
    kernels' arithmetic and not a weaker stand-in."""
    rng = np.random.default_rng(3)
    N = 700
    lens = rng.integers(1, 90, size=N)
    seg = np.repeat(np.arange(len(lens)), lens)[:N][None].astype(np.int32)
    s = seg[0]
    for causal in (True, False):
        vis = (s[:, None] == s[None, :]) & ((np.arange(N)[None, :] <= np.arange(N)[:, None]) | (not causal))
        for tile, other, keys in JOBS:
            tab = table(seg, tile, other, keys, causal)[0]
            m = vis.T if keys else vis          # rows: this table's tiles
            for it, (lo, hi) in enumerate(tab):
                rows = m[it * tile:min(it * tile + tile, N)].any(axis=0)
                cols = np.nonzero(rows)[0] // other
                assert lo == cols.min() and hi == cols.max()
