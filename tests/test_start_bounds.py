"""Bounds that the kernels' start sweeps and Hessian rely on (CPU only, numpy).

The Newton start is three Sinkhorn-Knopp sweeps (scale the columns of a
row-stochastic T to sum to one, renormalise the rows).  The kernels test the
column sums for underflow / NaN before the first sweep only, and form the
product of the later sweeps' ratios c_{n-1} / c_j before taking one logarithm.
Both rest on this fact: after one sweep every column sum is at least 1/n
(column j of T diag(1/c) holds weights v_i summing to one, and no row of it
sums to more than n, so the renormalised column sums to at least
sum_i v_i / n), and at most n, so every later ratio lies within [n^-2, n^2].
The Hessian diagonal of eq (9) ([P] section 3.2) is summed as sum_{k != j} G_jk over the column Gram sums
G_jk = sum_i T_ij T_ik, which equals c_j - sum_i T_ij^2 when rows sum to one.

Sources: "Accelerating Birkhoff Projection for Manifold-Constrained
Hyper-Connections", section 2.2 (eq 2, the Sinkhorn-Knopp sweep) and
section 3.2 (eq 9, the Hessian).
"""
import numpy as np
import pytest


def row_softmax(L):
    E = np.exp(L - L.max(axis=-1, keepdims=True))
    return E / E.sum(axis=-1, keepdims=True)


def sweep(T):
    """One Sinkhorn-Knopp sweep of a row-stochastic T: columns to one, rows renormalised."""
    c = T.sum(axis=-2, keepdims=True)
    U = T / c
    return U / U.sum(axis=-1, keepdims=True), c[..., 0, :]


def adversarial_logits(rng, B, n, dtype):
    """Normal logits at scales up to 30, and rows that put nearly all mass in one
    column (by e^40, or by e^100 so that the other columns underflow in fp32)."""
    sig = rng.choice([0.5, 3.0, 8.0, 30.0], size=(B, 1, 1))
    L = sig * rng.standard_normal((B, n, n))
    q = B // 4
    hot = rng.integers(0, n, size=(2 * q,))
    L[np.arange(q), :, hot[:q]] += 40.0
    L[np.arange(q, 2 * q), :, hot[q:]] += 100.0
    return L.astype(dtype)


@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_column_sums_after_one_sweep_are_at_least_one_over_n(n, dtype):
    rng = np.random.default_rng(11 + n)
    T = row_softmax(adversarial_logits(rng, 20000, n, dtype))
    c0 = T.sum(axis=-2)
    ok = (c0 > np.finfo(np.float32).tiny).all(axis=-1)   # the kernels' one test
    assert ok.mean() > 0.3 and (~ok).any()                # both branches occur in this sample
    T = T[ok]
    floor = 1.0 / n * (1 - 1e-5)
    for k in range(1, 4):                                 # sweeps 1, 2, 3
        T, c = sweep(T)
        cn = T.sum(axis=-2)
        assert cn.min() >= floor, (k, cn.min())
        if k >= 2:                                        # ratios of the later sweeps
            ratio = c[:, -1:] / c[:, :-1]
            assert ratio.min() >= n ** -2.0 * (1 - 1e-5) and ratio.max() <= n ** 2.0 * (1 + 1e-5)


def test_column_sum_floor_is_not_vacuous():
    """One row spread over every column, the others concentrated on column 1:
    after one sweep column 0 sums to about 0.32, above the floor 1/n = 0.25."""
    n, d = 4, 1e-9
    T = np.array([[0.25, 0.25, 0.25, 0.25]] + [[d, 1 - 3 * d, d, d]] * 3)
    T2, _ = sweep(T[None])
    cs = T2.sum(axis=-2)[0]
    assert cs.min() >= 1.0 / n
    assert cs.min() < 0.33


@pytest.mark.parametrize("n", [2, 4, 8])
def test_hessian_diagonal_from_gram_sums(n):
    rng = np.random.default_rng(5 + n)
    T = row_softmax(3.0 * rng.standard_normal((2000, n, n)))
    G = np.einsum("bij,bik->bjk", T, T)                   # column Gram sums, all n columns
    c = T.sum(axis=-2)
    for j in range(n - 1):
        gram_form = sum(G[:, j, k] for k in range(n) if k != j)
        plain = c[:, j] - (T[:, :, j] ** 2).sum(axis=-1)
        row_form = (T[:, :, j] * (T.sum(axis=-1) - T[:, :, j])).sum(axis=-1)
        np.testing.assert_allclose(gram_form, plain, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(gram_form, row_form, rtol=1e-12, atol=1e-15)
        assert (gram_form >= 0).all()


def test_gram_diagonal_keeps_relative_accuracy_in_fp32():
    """A column carried by one entry near 1: c_j - sum_i T_ij^2 cancels in fp32,
    the sum of non-negative Gram terms does not."""
    n = 4
    L = np.zeros((n, n))
    L[:, 0] = -30.0
    L[0, 0] = 30.0
    T64 = row_softmax(L)
    T32 = T64.astype(np.float32)
    exact = sum((T64[:, 0] * T64[:, k]).sum() for k in range(1, n))
    gram32 = np.float32(0)
    for k in range(1, n):
        gram32 += np.float32((T32[:, 0] * T32[:, k]).sum(dtype=np.float32))
    plain32 = T32[:, 0].sum(dtype=np.float32) - (T32[:, 0] * T32[:, 0]).sum(dtype=np.float32)
    assert abs(float(gram32) - exact) <= 1e-5 * exact
    assert abs(float(plain32) - exact) > 0.5 * exact       # cancellation loses it
