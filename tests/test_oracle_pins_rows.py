"""Pins of the oracle's row-subset gradient helpers, grad_h_rows and
grad_w_rows, the expected values of every sampled-gradient check at the large
workloads.

Both are checked against torch fp64 autograd of the plain definition
F = sum_t g_t log_softmax(z_t)[y_t] with g held fixed (so dF/dh_t, dF/dW_v and
dF/db_v are exactly the input, weight and bias gradients of the fused linear
layer that Liger PR #1320 "The implementation" lists), against central finite
differences of the same F computed with scipy's logsumexp, and against the
whole-batch backward(), itself pinned by finite differences and autograd in
tests/test_oracle_pins.py. A wrong sign, a dropped temperature, a mis-used
log-sum-exp or a transposed operand in either helper fails one of them.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _problem(seed, bias, tau, N=29, H=6, V=41):
    r = np.random.default_rng(seed)
    h = r.standard_normal((N, H))
    W = r.standard_normal((V, H)) * 0.6
    b = r.standard_normal(V) * 0.4 if bias else None
    y = r.integers(0, V, N)
    y[:4] = 7                       # several tokens share one target row
    g = r.standard_normal(N)
    g[[3, 11]] = 0.0                # tokens without a gradient
    return h, W, b, y, g


def _autograd(h, W, b, y, g, tau):
    """dF/dh, dF/dW, dF/db of F = sum_t g_t log_softmax((h W^T + b)/tau)[y_t]."""
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    bt = None if b is None else torch.tensor(b, dtype=torch.float64, requires_grad=True)
    z = ht @ Wt.T
    if bt is not None:
        z = z + bt
    lp = torch.log_softmax(z / tau, dim=1).gather(1, torch.as_tensor(y)[:, None])[:, 0]
    (torch.as_tensor(g) * lp).sum().backward()
    return ht.grad.numpy(), Wt.grad.numpy(), None if bt is None else bt.grad.numpy()


def _F(h, W, b, y, g, tau):
    z = h @ W.T
    if b is not None:
        z = z + b
    z = z / tau
    lp = z[np.arange(len(y)), y] - scipy.special.logsumexp(z, axis=1)
    return float((g * lp).sum())


CASES = [(False, 1.0), (True, 1.0), (False, 0.7), (True, 1.3)]


@pytest.mark.parametrize("bias,tau", CASES)
def test_grad_h_rows_against_autograd_and_backward(bias, tau):
    h, W, b, y, g = _problem(21, bias, tau)
    lse = oracle.forward_rows(h, W, b, tau, y)["lse"]
    gh_ad, _, _ = _autograd(h, W, b, y, g, tau)
    rows = np.array([0, 2, 3, 5, 11, 17, 28])
    got = oracle.grad_h_rows(h[rows], W, b, tau, y[rows], lse[rows], g[rows])
    np.testing.assert_allclose(got, gh_ad[rows], rtol=0, atol=1e-12)
    gh_bw, _, _ = oracle.backward(h, W, b, tau, y, lse, g, chunk=5)
    np.testing.assert_allclose(got, gh_bw[rows], rtol=0, atol=1e-12)
    assert np.all(got[[2, 4]] == 0)  # g = 0 rows (tokens 3 and 11)


@pytest.mark.parametrize("bias,tau", CASES)
@pytest.mark.parametrize("chunk", [1, 4, 7, 1000])
def test_grad_w_rows_against_autograd_and_backward(bias, tau, chunk):
    """Every chunk size that splits N = 29 unevenly (and one larger than N)
    gives the autograd gradient on the sampled rows, target rows included."""
    h, W, b, y, g = _problem(22, bias, tau)
    lse = oracle.forward_rows(h, W, b, tau, y)["lse"]
    _, gW_ad, gb_ad = _autograd(h, W, b, y, g, tau)
    vrows = np.array([0, 7, 13, int(y[20]), 40])
    gW, gb = oracle.grad_w_rows(h, W[vrows], None if b is None else b[vrows], tau, y, lse, g, vrows, chunk=chunk)
    np.testing.assert_allclose(gW, gW_ad[vrows], rtol=0, atol=1e-12)
    _, gW_bw, gb_bw = oracle.backward(h, W, b, tau, y, lse, g, chunk=6)
    np.testing.assert_allclose(gW, gW_bw[vrows], rtol=0, atol=1e-12)
    if b is not None:
        np.testing.assert_allclose(gb, gb_ad[vrows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gb, gb_bw[vrows], rtol=0, atol=1e-12)
    else:
        # the bias gradient is returned whether or not the layer has a bias
        np.testing.assert_allclose(gb, gb_bw[vrows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("bias,tau", [(True, 0.7), (False, 1.3)])
def test_row_helpers_finite_differences(bias, tau):
    """Central differences of F in fp64 on coordinates of W, b and h."""
    h, W, b, y, g = _problem(23, bias, tau)
    lse = oracle.forward_rows(h, W, b, tau, y)["lse"]
    vrows = np.array([2, 7, 30])
    gW, gb = oracle.grad_w_rows(h, W[vrows], None if b is None else b[vrows], tau, y, lse, g, vrows, chunk=9)
    rows = np.array([1, 6, 20])
    gh = oracle.grad_h_rows(h[rows], W, b, tau, y[rows], lse[rows], g[rows])
    d = 1e-6
    r = np.random.default_rng(24)

    def cdiff(arr, idx):
        s = arr[idx]
        arr[idx] = s + d
        fp = _F(h, W, b, y, g, tau)
        arr[idx] = s - d
        fm = _F(h, W, b, y, g, tau)
        arr[idx] = s
        return (fp - fm) / (2 * d)

    for k, v in enumerate(vrows):
        for j in r.choice(W.shape[1], 3, replace=False):
            assert gW[k, j] == pytest.approx(cdiff(W, (v, j)), rel=1e-6, abs=1e-9)
        if b is not None:
            assert gb[k] == pytest.approx(cdiff(b, (v,)), rel=1e-6, abs=1e-9)
    for k, t in enumerate(rows):
        for j in r.choice(h.shape[1], 3, replace=False):
            assert gh[k, j] == pytest.approx(cdiff(h, (t, j)), rel=1e-6, abs=1e-9)


def test_grad_w_rows_vocabulary_sums_vanish():
    """Summed over every vocabulary row, sum_v dz[t,v] = g_t (1 - sum_v p) / tau = 0,
    so the full set of rows sums to zero (the property the largest workload's
    check leans on)."""
    h, W, b, y, g = _problem(25, True, 0.9)
    lse = oracle.forward_rows(h, W, b, 0.9, y)["lse"]
    vrows = np.arange(W.shape[0])
    gW, gb = oracle.grad_w_rows(h, W, b, 0.9, y, lse, g, vrows, chunk=8)
    np.testing.assert_allclose(gW.sum(0), 0.0, atol=1e-12)
    assert abs(gb.sum()) < 1e-12
