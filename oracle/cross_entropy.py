"""fp64 CPU oracle for the fused linear cross-entropy loss.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The HIP library
never calls it and shares no code with it.

What it computes is the plain definition, with the logits written out in full
(the thing the fused kernel exists to avoid):

* Forward.  For hidden states H (N, D), a dense output head W (V, D) and
  integer targets t (N,), the logits are Z = H W^T (N, V).  Per token the loss
  layer returns three N-length arrays, as the mlx-train-perf README states for
  its fused loss (section "The fused cross-entropy loss"): the log-sum-exp
  LSE_i = ln sum_v exp(Z_iv) (computed stably by subtracting the row max), the
  target logit Z_{i, t_i}, and the negative log-likelihood
  NLL_i = LSE_i - Z_{i, t_i}.

* Backward, from per-token upstream gradients g_i = dLoss/dNLL_i (a mean
  reduction is g_i = 1/N):
      dZ = g_i (softmax(Z_i) - onehot(t_i))     row by row
      dH = dZ W,  dW = dZ^T H
  The pages do not print these formulas; they are the chain rule through
  log-softmax.

All arithmetic is float64 on the exact values the GPU receives.  Rows are
processed in blocks purely to bound memory.
"""
from __future__ import annotations

import numpy as np

__all__ = ["lce_forward", "lce_backward", "lce_rows"]


def _check(h, w, targets):
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w)                 # converted to float64 a block of rows at a time
    t = np.asarray(targets, dtype=np.int64)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1] or t.shape != (h.shape[0],):
        raise ValueError("expected h (N, D), w (V, D), targets (N,)")
    if t.size and (t.min() < 0 or t.max() >= w.shape[0]):
        raise ValueError("targets must lie in [0, V)")
    return h, w, t


def _logits(hr, w, vocab_block=16384):
    """hr (R, D) float64 times w^T, w converted to float64 in row blocks."""
    z = np.empty((hr.shape[0], w.shape[0]))
    for v0 in range(0, w.shape[0], vocab_block):
        z[:, v0:v0 + vocab_block] = hr @ np.asarray(w[v0:v0 + vocab_block], dtype=np.float64).T
    return z


def _block(h, w, t, rows):
    z = _logits(h[rows], w)
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    tz = z[np.arange(rows.size), t[rows]]
    return z, lse, tz


def lce_forward(h, w, targets, row_block=1024):
    """(NLL, LSE, target logit), each (N,) float64."""
    h, w, t = _check(h, w, targets)
    N = h.shape[0]
    nll, lse, tz = (np.empty(N) for _ in range(3))
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(r0 + row_block, N))
        _, l, z_t = _block(h, w, t, rows)
        lse[rows], tz[rows] = l, z_t
        nll[rows] = l - z_t
    return nll, lse, tz


def lce_backward(h, w, targets, g, row_block=1024):
    """dH (N, D) and dW (V, D), float64, for upstream gradients g (N,)."""
    h, w, t = _check(h, w, targets)
    g = np.asarray(g, dtype=np.float64)
    N = h.shape[0]
    w64 = np.asarray(w, dtype=np.float64)
    dh = np.empty_like(h)
    dw = np.zeros_like(w64)
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(r0 + row_block, N))
        z, l, _ = _block(h, w64, t, rows)
        dz = np.exp(z - l[:, None])
        dz[np.arange(rows.size), t[rows]] -= 1.0
        dz *= g[rows][:, None]
        dh[rows] = dz @ w64
        dw += dz.T @ h[rows]
    return dh, dw


def lce_rows(h, w, targets, g, rows):
    """For selected tokens only: NLL, LSE, target logit and dH rows (sampled
    checks at sizes where the full logits do not fit)."""
    h, w, t = _check(h, w, targets)
    g = np.asarray(g, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    z, l, z_t = _block(h, w, t, rows)
    dz = np.exp(z - l[:, None])
    dz[np.arange(rows.size), t[rows]] -= 1.0
    dz *= g[rows][:, None]
    dh = np.zeros((rows.size, h.shape[1]))
    for v0 in range(0, w.shape[0], 16384):
        dh += dz[:, v0:v0 + 16384] @ np.asarray(w[v0:v0 + 16384], dtype=np.float64)
    return l - z_t, l, z_t, dh
