"""Pins for the fp64 linear cross-entropy oracle (CPU only).

* a hand-derived example (values worked on paper from the definition);
* closed forms (identical head rows give a uniform softmax);
* central finite differences of sum(g * NLL) for dH and dW;
* an exact identity (every row of dZ sums to zero, so sum_v dW_v = 0);
* PyTorch CPU fp64 cross_entropy + autograd as a library cross-check.
"""
import math

import numpy as np
import pytest

from oracle import lce_backward, lce_forward, lce_rows


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_derived_example():
    # one token, D = 1, h = 1, head rows 0, ln 2, ln 3: logits 0, ln 2, ln 3,
    # exp-sum 1 + 2 + 3 = 6; target 2
    h = np.array([[1.0]])
    w = np.array([[0.0], [math.log(2.0)], [math.log(3.0)]])
    t = np.array([2])
    nll, lse, tz = lce_forward(h, w, t)
    assert lse[0] == pytest.approx(math.log(6.0), abs=1e-15)
    assert tz[0] == pytest.approx(math.log(3.0), abs=1e-15)
    assert nll[0] == pytest.approx(math.log(2.0), abs=1e-15)
    # softmax (1/6, 2/6, 3/6) minus onehot(2): dZ = (1/6, 1/3, -1/2)
    dh, dw = lce_backward(h, w, t, np.array([1.0]))
    assert dh[0, 0] == pytest.approx(math.log(2.0) / 3.0 - math.log(3.0) / 2.0, abs=1e-15)
    np.testing.assert_allclose(dw[:, 0], [1 / 6, 1 / 3, -1 / 2], rtol=0, atol=1e-15)


def test_identical_head_rows():
    """All V head rows equal: softmax is uniform, NLL = ln V, dH = 0 and
    dW_v = g (1/V - [v = t]) h."""
    N, V, D = 5, 7, 4
    h = _rand((N, D), 1)
    w = np.tile(_rand((1, D), 2), (V, 1))
    t = np.array([0, 3, 6, 6, 2])
    g = _rand(N, 3)
    nll, lse, tz = lce_forward(h, w, t)
    np.testing.assert_allclose(nll, np.full(N, math.log(V)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, h @ w[0] + math.log(V), rtol=0, atol=1e-13)
    dh, dw = lce_backward(h, w, t, g)
    assert np.abs(dh).max() < 1e-13
    expect = np.zeros((V, D))
    for i in range(N):
        expect += g[i] * (np.full((V, 1), 1.0 / V) - (np.arange(V) == t[i])[:, None]) * h[i]
    np.testing.assert_allclose(dw, expect, rtol=0, atol=1e-13)


@pytest.mark.parametrize("N,V,D", [(1, 3, 2), (3, 5, 4), (4, 9, 3)])
def test_finite_differences(N, V, D):
    h, w, g = _rand((N, D), 10 + N), _rand((V, D), 20 + V), _rand(N, 30 + D)
    t = np.random.default_rng(40).integers(0, V, N)
    dh, dw = lce_backward(h, w, t, g)
    step = 1e-6

    def loss():
        return float(np.sum(g * lce_forward(h, w, t)[0]))

    for x, grad in ((h, dh), (w, dw)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + step
            lp = loss()
            x[idx] = old - step
            lm = loss()
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * step)
        assert np.abs(fd - grad).max() / max(1.0, np.abs(grad).max()) < 1e-7


def test_dw_rows_sum_to_zero_and_bounds():
    N, V, D = 30, 50, 8
    h, w = _rand((N, D), 50), _rand((V, D), 51) * 2
    t = np.random.default_rng(52).integers(0, V, N)
    g = _rand(N, 53)
    nll, lse, tz = lce_forward(h, w, t)
    assert (nll >= 0).all() and (tz <= lse).all()
    _, dw = lce_backward(h, w, t, g)
    assert np.abs(dw.sum(axis=0)).max() < 1e-12


def test_rows_helper_matches_full():
    N, V, D = 20, 40, 6
    h, w = _rand((N, D), 60), _rand((V, D), 61)
    t = np.random.default_rng(62).integers(0, V, N)
    g = _rand(N, 63)
    nll, lse, tz = lce_forward(h, w, t)
    dh, _ = lce_backward(h, w, t, g)
    rows = np.array([0, 7, 19])
    r_nll, r_lse, r_tz, r_dh = lce_rows(h, w, t, g, rows)
    np.testing.assert_allclose(r_nll, nll[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r_lse, lse[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r_tz, tz[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r_dh, dh[rows], rtol=0, atol=1e-13)
    # row blocking does not change results
    for a, b in zip(lce_forward(h, w, t, row_block=7), (nll, lse, tz)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_refuses_bad_targets():
    with pytest.raises(ValueError):
        lce_forward(np.zeros((2, 3)), np.zeros((4, 3)), np.array([0, 4]))
    with pytest.raises(ValueError):
        lce_forward(np.zeros((2, 3)), np.zeros((4, 2)), np.array([0, 1]))


def test_against_torch_cross_entropy_fp64():
    torch = pytest.importorskip("torch")
    N, V, D = 12, 33, 10
    h, w = _rand((N, D), 70), _rand((V, D), 71)
    t = np.random.default_rng(72).integers(0, V, N)
    g = _rand(N, 73)
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    logits = th @ tw.T
    nll_t = torch.nn.functional.cross_entropy(logits, torch.tensor(t), reduction="none")
    (nll_t * torch.tensor(g)).sum().backward()
    nll, lse, tz = lce_forward(h, w, t)
    np.testing.assert_allclose(nll, nll_t.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, 1).detach().numpy(), rtol=1e-12, atol=1e-12)
    dh, dw = lce_backward(h, w, t, g)
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-11, atol=1e-11)
