"""fp64 CPU oracle for O(N)-memory attention: forward, log-sum-exp and backward.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The HIP library
never calls it and shares no code with it.

What it computes is the plain definition, written out with an explicit
visibility mask over all N keys (no tile skipping, no online softmax):

* Visibility.  Query i sees key j when j <= i (causal) and, for packed rows,
  when both tokens carry the same segment id.  This is the block-diagonal causal
  rule of the mlx-train-perf 0.5.1 README, section "Sequence packing" (a token
  attends another only when both come from the same original sequence), driven
  by a per-token segment id as in the mlx-train-perf changelog, section "Added"
  (the PACKED kernel variant).  With causal off and a segment id given, the mask
  is segment equality alone (block-diagonal, bidirectional).

* Forward.  S = scale * Q K^T, masked entries set to -inf, LSE_i the natural
  log of sum_j exp(S_ij) (computed stably by subtracting the row max),
  P = exp(S - LSE), O = P V.  O and LSE are the saved state the README's
  "Flash-attention training path" section names (the attention output and the
  log-sum-exp).

* Backward, from the loss gradient dO alone (no gradient flows into LSE):
      dP = dO V^T
      Dr_i = sum_d dO_id O_id          (= sum_j P_ij dP_ij, since O = P V)
      dS = P * (dP - Dr)               (softmax Jacobian applied row by row)
      dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
  The pages do not print these formulas; they say only that the backward
  recomputes the tiles it needs from the saved state.  They follow from the
  chain rule through softmax: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik).

* Grouped-query heads.  K and V may carry Hkv heads for H query heads (H a
  multiple of Hkv); query head h then reads key/value head h // (H / Hkv), the
  groups being contiguous runs of query heads as the mlx-train-perf README
  states for its attention op (section "If you maintain a trainer": grouped
  query heads mapped contiguously).  dK and dV of a key/value head are sums
  over the query heads that read it.

All arithmetic is float64 on the exact values the GPU receives.  Rows are
processed in blocks of ``row_block`` queries purely to bound memory; each block
still builds the explicit mask over every key.
"""
from __future__ import annotations

import numpy as np

__all__ = ["visible_mask", "attention_forward", "attention_backward",
           "attention_rows", "attention_backward_rows", "visible_pairs"]


def visible_mask(rows: np.ndarray, N: int, seg_row: np.ndarray | None,
                 causal: bool) -> np.ndarray:
    """Boolean (len(rows), N) mask: True where query rows[r] may see key j."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(N, dtype=np.int64)
    m = np.ones((rows.size, N), dtype=bool)
    if causal:
        m &= j[None, :] <= rows[:, None]
    if seg_row is not None:
        seg_row = np.asarray(seg_row)
        m &= seg_row[rows][:, None] == seg_row[None, :]
    return m


def _scores(qr: np.ndarray, k: np.ndarray, scale: float, mask: np.ndarray) -> np.ndarray:
    s = scale * (qr @ k.T)
    s[~mask] = -np.inf
    return s


def _row_lse(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=1)
    # every row has at least one visible key (the diagonal), so m is finite
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def _group(q, k):
    """Query heads per key/value head."""
    H, Hkv = q.shape[1], k.shape[1]
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"{H} query heads do not split into groups over {Hkv} key/value heads")
    return H // Hkv


def attention_forward(q, k, v, seg=None, scale=None, causal=True, row_block=512):
    """O (B,H,N,D) and LSE (B,H,N), float64.  ``seg`` is (B,N) ints or None;
    k and v are (B,Hkv,N,D) with Hkv dividing H."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    G = _group(q, k)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    scale = float(scale)
    o = np.empty((B, H, N, D), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        seg_row = None if seg is None else np.asarray(seg)[b]
        for r0 in range(0, N, row_block):
            rows = np.arange(r0, min(r0 + row_block, N))
            mask = visible_mask(rows, N, seg_row, causal)
            for h in range(H):
                g = h // G
                s = _scores(q[b, h, rows], k[b, g], scale, mask)
                l = _row_lse(s)
                p = np.exp(s - l[:, None])
                o[b, h, rows] = p @ v[b, g]
                lse[b, h, rows] = l
    return o, lse


def attention_backward(q, k, v, do, seg=None, scale=None, causal=True,
                       o=None, lse=None, row_block=512):
    """dQ (B,H,N,D), dK and dV (B,Hkv,N,D), float64, for loss gradient ``do``.

    O and LSE are the oracle's own fp64 forward results; they are recomputed
    when not passed in.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, D = q.shape
    G = _group(q, k)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    scale = float(scale)
    if o is None or lse is None:
        o, lse = attention_forward(q, k, v, seg, scale, causal, row_block)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        seg_row = None if seg is None else np.asarray(seg)[b]
        for r0 in range(0, N, row_block):
            rows = np.arange(r0, min(r0 + row_block, N))
            mask = visible_mask(rows, N, seg_row, causal)
            for h in range(H):
                g = h // G
                s = _scores(q[b, h, rows], k[b, g], scale, mask)
                p = np.exp(s - lse[b, h, rows][:, None])
                dp = do[b, h, rows] @ v[b, g].T
                dr = np.sum(do[b, h, rows] * o[b, h, rows], axis=1)
                ds = p * (dp - dr[:, None])
                dq[b, h, rows] = scale * (ds @ k[b, g])
                dk[b, g] += scale * (ds.T @ q[b, h, rows])
                dv[b, g] += p.T @ do[b, h, rows]
    return dq, dk, dv


def attention_rows(q_bh, k_bh, v_bh, rows, seg_row=None, scale=None, causal=True):
    """O and LSE of selected query rows of one (batch, head): for sampled checks.

    ``q_bh``, ``k_bh``, ``v_bh`` are (N, D); returns (O rows (R, D), LSE (R,)).
    """
    q_bh = np.asarray(q_bh, dtype=np.float64)
    k_bh = np.asarray(k_bh, dtype=np.float64)
    v_bh = np.asarray(v_bh, dtype=np.float64)
    N, D = k_bh.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    mask = visible_mask(rows, N, seg_row, causal)
    s = _scores(q_bh[rows], k_bh, float(scale), mask)
    l = _row_lse(s)
    p = np.exp(s - l[:, None])
    return p @ v_bh, l


def attention_backward_rows(q_bh, k_bh, v_bh, do_bh, o_rows, lse_rows, rows, seg_row=None,
                            scale=None, causal=True):
    """The backward restricted to selected query rows of one (batch, head).

    Returns dQ of those rows and the contributions those rows make to dK and
    dV (full (N, D) arrays); summed over a partition of all rows they give
    attention_backward's dK and dV.  ``o_rows``/``lse_rows`` are the rows' O
    and LSE from attention_rows.
    """
    q_bh = np.asarray(q_bh, dtype=np.float64)
    k_bh = np.asarray(k_bh, dtype=np.float64)
    v_bh = np.asarray(v_bh, dtype=np.float64)
    do_bh = np.asarray(do_bh, dtype=np.float64)
    N, D = k_bh.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    scale = float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    mask = visible_mask(rows, N, seg_row, causal)
    s = _scores(q_bh[rows], k_bh, scale, mask)
    p = np.exp(s - np.asarray(lse_rows, dtype=np.float64)[:, None])
    dp = do_bh[rows] @ v_bh.T
    dr = np.sum(do_bh[rows] * np.asarray(o_rows, dtype=np.float64), axis=1)
    ds = p * (dp - dr[:, None])
    return scale * (ds @ k_bh), scale * (ds.T @ q_bh[rows]), p.T @ do_bh[rows]


def visible_pairs(N: int, seg_row: np.ndarray | None, causal: bool = True) -> int:
    """Number of visible (query, key) pairs of one (batch, head), counted directly."""
    total = 0
    for r0 in range(0, N, 1024):
        rows = np.arange(r0, min(r0 + 1024, N))
        total += int(visible_mask(rows, N, seg_row, causal).sum())
    return total
