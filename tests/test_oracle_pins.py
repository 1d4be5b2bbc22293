"""Pins for the fp64 oracle, each independent of the oracle's own code path.

* hand-derived values (tests/golden/hand_n3_d1.json, worked out on paper);
* closed forms (one key, length-1 segments, equal keys, constant values);
* central finite differences of the loss sum(dO * O) for every gradient;
* invariants that hold exactly in real arithmetic (packed row == each segment
  alone, per-segment gradient sums, the Q.dQ == K.dK identity);
* PyTorch's CPU fp64 scaled_dot_product_attention plus autograd, as a library
  cross-check on small shapes.
"""
import json
import os

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_rows, attention_forward,
                    attention_rows, visible_mask, visible_pairs)
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_n3_d1.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _as4(x):
    """(N, D) list -> (1, 1, N, D) float64."""
    return np.asarray(x, dtype=np.float64)[None, None]


# ---------------------------------------------------------------- hand values

def _golden_cases():
    with open(GOLDEN) as f:
        g = json.load(f)
    return g["inputs"], g["cases"]


@pytest.mark.parametrize("case_idx", range(4))
def test_hand_derived_example(case_idx):
    inp, cases = _golden_cases()
    c = cases[case_idx]
    q, k, v, do = (_as4(inp["q"]), _as4(inp["k"]["value"]), _as4(inp["v"]), _as4(inp["do"]))
    seg = None if c["seg"] is None else np.asarray([c["seg"]], dtype=np.int32)
    o, lse = attention_forward(q, k, v, seg, inp["scale"], c["causal"])
    dq, dk, dv = attention_backward(q, k, v, do, seg, inp["scale"], c["causal"])
    np.testing.assert_allclose(o[0, 0, :, 0], c["o"]["value"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], c["lse"]["value"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq[0, 0, :, 0], c["dq"]["value"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk[0, 0, :, 0], c["dk"]["value"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv[0, 0, :, 0], c["dv"]["value"], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [True, False])
def test_single_token(causal):
    """N = 1: the one key is the only one visible, so P = 1."""
    B, H, D = 2, 3, 8
    q, k, v, do = (_rand((B, H, 1, D), s) for s in range(4))
    scale = 0.37
    o, lse = attention_forward(q, k, v, None, scale, causal)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, scale * np.sum(q * k, axis=-1), rtol=0, atol=1e-14)
    dq, dk, dv = attention_backward(q, k, v, do, None, scale, causal)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


def test_length_one_segments():
    """Every token its own segment: each query sees only itself."""
    B, H, N, D = 1, 2, 7, 4
    q, k, v, do = (_rand((B, H, N, D), 10 + s) for s in range(4))
    seg = np.arange(N, dtype=np.int32)[None]
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, seg, 0.5, causal)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, 0.5 * np.sum(q * k, axis=-1), rtol=0, atol=1e-14)
        dq, dk, dv = attention_backward(q, k, v, do, seg, 0.5, causal)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
        np.testing.assert_allclose(dv, do, rtol=0, atol=1e-14)


def test_equal_keys_give_uniform_average():
    """All keys of a segment equal: P is uniform over the visible keys."""
    N, D = 9, 5
    seg = np.array([[0, 0, 0, 0, 1, 1, 1, 1, 1]], dtype=np.int32)
    kvec = np.array([0.3, -1.2, 0.5, 2.0, -0.7])
    k = np.tile(kvec, (N, 1))[None, None]
    q = _rand((1, 1, N, D), 21)
    v = _rand((1, 1, N, D), 22)
    do = _rand((1, 1, N, D), 23)
    scale = 0.8
    o, lse = attention_forward(q, k, v, seg, scale, True)
    dq, _, _ = attention_backward(q, k, v, do, seg, scale, True)
    for i in range(N):
        start = 0 if seg[0, i] == 0 else 4
        vis = np.arange(start, i + 1)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, vis].mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], scale * q[0, 0, i] @ kvec + np.log(vis.size),
                                   rtol=0, atol=1e-13)
    assert np.abs(dq).max() < 1e-13


def test_constant_values():
    """V rows all equal to c: O = c everywhere and no gradient reaches Q or K."""
    B, H, N, D = 1, 2, 11, 6
    q, k, do = (_rand((B, H, N, D), 30 + s) for s in range(3))
    c = np.linspace(-1, 2, D)
    v = np.broadcast_to(c, (B, H, N, D)).copy()
    seg = workloads.random_segments(B, N, 3)
    for s in (None, seg):
        o, _ = attention_forward(q, k, v, s, 0.4, True)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)
        dq, dk, _ = attention_backward(q, k, v, do, s, 0.4, True)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


# ---------------------------------------------------------------- finite differences

def _loss(q, k, v, do, seg, scale, causal):
    o, _ = attention_forward(q, k, v, seg, scale, causal)
    return float(np.sum(do * o))


@pytest.mark.parametrize("N,D,causal,packed", [
    (1, 4, True, False), (2, 4, True, True), (5, 8, True, True),
    (16, 4, True, True), (16, 8, True, False), (5, 4, False, True), (6, 4, False, False),
])
def test_finite_differences(N, D, causal, packed):
    B, H = 1, 2
    q, k, v, do = (_rand((B, H, N, D), 100 * N + D + s) for s in range(4))
    seg = workloads.random_segments(B, N, N, max_len=3) if packed else None
    scale = 1.0 / np.sqrt(D)
    grads = attention_backward(q, k, v, do, seg, scale, causal)
    h = 1e-6
    for x, g in zip((q, k, v), grads):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, seg, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, seg, scale, causal)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, err


@pytest.mark.parametrize("Hkv,causal,packed", [(2, True, False), (1, True, True), (2, False, True)])
def test_finite_differences_grouped_heads(Hkv, causal, packed):
    """Grouped-query heads: 4 query heads over Hkv key/value heads."""
    B, H, N, D = 1, 4, 5, 4
    q, do = (_rand((B, H, N, D), 300 + s) for s in range(2))
    k, v = (_rand((B, Hkv, N, D), 310 + s) for s in range(2))
    seg = workloads.random_segments(B, N, 7, max_len=3) if packed else None
    scale = 0.45
    grads = attention_backward(q, k, v, do, seg, scale, causal)
    assert grads[1].shape == k.shape and grads[2].shape == v.shape
    h = 1e-6
    for x, g in zip((q, k, v), grads):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, seg, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, seg, scale, causal)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, err


def test_grouped_heads_refuse_uneven_groups():
    q = np.zeros((1, 4, 3, 4))
    k = np.zeros((1, 3, 3, 4))
    with pytest.raises(ValueError):
        attention_forward(q, k, k)


# ---------------------------------------------------------------- invariants

def test_packed_row_equals_segments_alone():
    """A packed row gives each segment exactly what it gets when run alone."""
    B, H, N, D = 2, 2, 40, 8
    q, k, v, do = (_rand((B, H, N, D), 40 + s) for s in range(4))
    seg = workloads.random_segments(B, N, 5, max_len=12)
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, seg, 0.3, causal)
        dq, dk, dv = attention_backward(q, k, v, do, seg, 0.3, causal)
        for b in range(B):
            start = 0
            for L in workloads.segment_lengths(seg[b]):
                sl = slice(start, start + L)
                args = [x[b:b + 1, :, sl] for x in (q, k, v)]
                o1, lse1 = attention_forward(*args, None, 0.3, causal)
                g1 = attention_backward(*args, do[b:b + 1, :, sl], None, 0.3, causal)
                np.testing.assert_allclose(o[b:b + 1, :, sl], o1, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(lse[b:b + 1, :, sl], lse1, rtol=1e-12, atol=1e-13)
                for ga, gb in zip((dq, dk, dv), g1):
                    np.testing.assert_allclose(ga[b:b + 1, :, sl], gb, rtol=1e-12, atol=1e-12)
                start += L


def test_single_segment_equals_plain_causal():
    B, H, N, D = 1, 2, 33, 8
    q, k, v, do = (_rand((B, H, N, D), 50 + s) for s in range(4))
    seg = np.zeros((B, N), dtype=np.int32)
    a = attention_forward(q, k, v, seg, 0.25, True) + attention_backward(q, k, v, do, seg, 0.25, True)
    b = attention_forward(q, k, v, None, 0.25, True) + attention_backward(q, k, v, do, None, 0.25, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # and the mask itself is the lower triangle
    assert np.array_equal(visible_mask(np.arange(N), N, seg[0], True), np.tril(np.ones((N, N), bool)))


def test_gradient_sums_per_segment():
    """Softmax shift invariance: sum of dK over a segment is 0; rows of P sum to 1."""
    B, H, N, D = 1, 3, 50, 8
    q, k, v, do = (_rand((B, H, N, D), 60 + s) for s in range(4))
    seg = workloads.random_segments(B, N, 6, max_len=15)
    dq, dk, dv = attention_backward(q, k, v, do, seg, 0.35, True)
    start = 0
    for L in workloads.segment_lengths(seg[0]):
        sl = slice(start, start + L)
        assert np.abs(dk[0, :, sl].sum(axis=1)).max() < 1e-12
        np.testing.assert_allclose(dv[0, :, sl].sum(axis=1), do[0, :, sl].sum(axis=1),
                                   rtol=0, atol=1e-12)
        start += L
    # sum_i q_i . dQ_i == sum_j k_j . dK_j  (both equal sum dS * scale QK^T)
    lhs = np.sum(q * dq, axis=(2, 3))
    rhs = np.sum(k * dk, axis=(2, 3))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_rows_helper_matches_forward():
    B, H, N, D = 1, 1, 70, 8
    q, k, v = (_rand((B, H, N, D), 70 + s) for s in range(3))
    seg = workloads.random_segments(B, N, 7, max_len=20)
    o, lse = attention_forward(q, k, v, seg, 0.3, True, row_block=16)
    rows = np.array([0, 5, 17, 69])
    o_r, lse_r = attention_rows(q[0, 0], k[0, 0], v[0, 0], rows, seg[0], 0.3, True)
    np.testing.assert_allclose(o_r, o[0, 0, rows], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse_r, lse[0, 0, rows], rtol=1e-14, atol=1e-14)


def test_backward_rows_partition_sums_to_full():
    """dQ rows and the per-row-block dK/dV contributions add up to the full backward."""
    B, H, N, D = 1, 1, 45, 8
    q, k, v, do = (_rand((B, H, N, D), 85 + s) for s in range(4))
    seg = workloads.random_segments(B, N, 85, max_len=20)
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, seg, 0.3, causal)
        dq, dk, dv = attention_backward(q, k, v, do, seg, 0.3, causal)
        dk_sum, dv_sum = np.zeros((N, D)), np.zeros((N, D))
        for rows in (np.arange(0, 10), np.arange(10, 31), np.arange(31, 45)):
            o_r, l_r = attention_rows(q[0, 0], k[0, 0], v[0, 0], rows, seg[0], 0.3, causal)
            dq_r, dk_r, dv_r = attention_backward_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], o_r, l_r,
                                                       rows, seg[0], 0.3, causal)
            np.testing.assert_allclose(dq_r, dq[0, 0, rows], rtol=1e-12, atol=1e-13)
            dk_sum += dk_r
            dv_sum += dv_r
        np.testing.assert_allclose(dk_sum, dk[0, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv_sum, dv[0, 0], rtol=1e-12, atol=1e-13)


def test_row_block_does_not_change_results():
    B, H, N, D = 1, 2, 37, 8
    q, k, v, do = (_rand((B, H, N, D), 80 + s) for s in range(4))
    seg = workloads.random_segments(B, N, 8)
    a = attention_backward(q, k, v, do, seg, 0.3, True, row_block=5)
    b = attention_backward(q, k, v, do, seg, 0.3, True, row_block=64)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)


def test_visible_pairs_closed_form():
    N = 300
    assert visible_pairs(N, None) == N * (N + 1) // 2
    seg = workloads.random_segments(1, N, 9, max_len=40)[0]
    lens = workloads.segment_lengths(seg)
    assert visible_pairs(N, seg) == sum(L * (L + 1) // 2 for L in lens)
    assert visible_pairs(N, seg, causal=False) == sum(L * L for L in lens)


def test_gradient_sums_per_segment_grouped_heads():
    """With K/V shared by a group of query heads, dK of a key/value head still
    sums to 0 over each segment, and dV sums to the group's summed dO."""
    B, H, Hkv, N, D = 1, 6, 2, 40, 8
    q, do = (_rand((B, H, N, D), 320 + s) for s in range(2))
    k, v = (_rand((B, Hkv, N, D), 330 + s) for s in range(2))
    seg = workloads.random_segments(B, N, 8, max_len=12)
    dq, dk, dv = attention_backward(q, k, v, do, seg, 0.3, True)
    grouped_do = do.reshape(B, Hkv, H // Hkv, N, D).sum(axis=2)
    start = 0
    for L in workloads.segment_lengths(seg[0]):
        sl = slice(start, start + L)
        assert np.abs(dk[0, :, sl].sum(axis=1)).max() < 1e-12
        np.testing.assert_allclose(dv[0, :, sl].sum(axis=1), grouped_do[0, :, sl].sum(axis=1),
                                   rtol=0, atol=1e-12)
        start += L


# ---------------------------------------------------------------- library cross-check

def test_against_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    B, H, N, D = 2, 2, 24, 8
    q, k, v, do = (_rand((B, H, N, D), 90 + s) for s in range(4))
    seg = workloads.random_segments(B, N, 11, max_len=9)
    scale = 0.3
    for causal in (True, False):
        for s in (None, seg):
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
            if s is None:
                mask = None
                is_causal = causal
            else:
                m = np.stack([visible_mask(np.arange(N), N, s[b], causal) for b in range(B)])
                mask = torch.tensor(m[:, None])
                is_causal = False
            if mask is None and not is_causal:
                out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
            else:
                out = torch.nn.functional.scaled_dot_product_attention(
                    tq, tk, tv, attn_mask=mask, is_causal=is_causal, scale=scale)
            out.backward(torch.tensor(do, dtype=torch.float64))
            o, _ = attention_forward(q, k, v, s, scale, causal)
            dq, dk, dv = attention_backward(q, k, v, do, s, scale, causal)
            np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_grouped_heads_against_torch_sdpa_fp64():
    """torch's SDPA with enable_gqa repeats each key/value head over a
    contiguous run of query heads, the convention the oracle follows."""
    torch = pytest.importorskip("torch")
    if "enable_gqa" not in (torch.nn.functional.scaled_dot_product_attention.__doc__ or ""):
        pytest.skip("this torch has no grouped-query SDPA")
    B, H, Hkv, N, D = 2, 6, 2, 20, 8
    q, do = (_rand((B, H, N, D), 340 + s) for s in range(2))
    k, v = (_rand((B, Hkv, N, D), 350 + s) for s in range(2))
    scale = 0.3
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale,
                                                           enable_gqa=True)
    out.backward(torch.tensor(do, dtype=torch.float64))
    o, _ = attention_forward(q, k, v, None, scale, True)
    dq, dk, dv = attention_backward(q, k, v, do, None, scale, True)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-11)
