"""Pins for the float64 oracle's mHC consumer step (CPU only): the residual-stream
mixing y = H_res x of the layer update x_{l+1} = H_res x_l + H_post^T F(H_pre x_l)
("Accelerating Birkhoff Projection for Manifold-Constrained Hyper-Connections",
section 2.1), with H_res the projected matrix T, and its backward.

Expected values come from numpy / torch routines the oracle does not use, from
exact properties of doubly stochastic and permutation matrices, and from finite
differences through the (separately pinned) projection."""
import numpy as np
import pytest

import oracle


def ds(rng, B, n):
    H = rng.standard_normal((B, n, n))
    T, _, _ = oracle.project(H)
    return H, T


@pytest.mark.parametrize("n,C", [(4, 1), (4, 37), (8, 64), (2, 5)])
def test_mix_matches_library_matmul(n, C):
    rng = np.random.default_rng(200 + n * C)
    T = rng.standard_normal((6, n, n))
    x = rng.standard_normal((6, n, C))
    np.testing.assert_allclose(oracle.mix(T, x), np.matmul(T, x), rtol=0, atol=1e-13)
    dy = rng.standard_normal((6, n, C))
    dx, dT = oracle.mix_bwd(T, x, dy)
    np.testing.assert_allclose(dx, np.einsum("bij,bic->bjc", T, dy), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dT, np.einsum("bic,bjc->bij", dy, x), rtol=0, atol=1e-12)


def test_doubly_stochastic_mixing_conserves_and_preserves():
    """Columns of a doubly stochastic T sum to one, so every column of y keeps the sum
    of the streams (1^T y = 1^T x); rows sum to one, so identical streams stay
    unchanged ([P] section 2.1: the mapping conserves the mean signal)."""
    rng = np.random.default_rng(201)
    _, T = ds(rng, 32, 4)
    x = rng.standard_normal((32, 4, 50))
    y = oracle.mix(T, x)
    np.testing.assert_allclose(y.sum(1), x.sum(1), rtol=0, atol=1e-12)
    v = rng.standard_normal((32, 1, 50))
    np.testing.assert_allclose(oracle.mix(T, np.repeat(v, 4, axis=1)), np.repeat(v, 4, axis=1), rtol=0, atol=1e-12)


def test_permutation_mixing_is_exact():
    rng = np.random.default_rng(202)
    x = rng.standard_normal((5, 4, 9))
    for q in range(5):
        perm = rng.permutation(4)
        P = np.eye(4)[perm][None]
        np.testing.assert_array_equal(oracle.mix(P, x[q:q + 1])[0], x[q, perm])


def test_mix_backward_matches_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(203)
    T0 = rng.standard_normal((4, 4, 4))
    x0 = rng.standard_normal((4, 4, 33))
    dy = rng.standard_normal((4, 4, 33))
    T = torch.tensor(T0, requires_grad=True)
    x = torch.tensor(x0, requires_grad=True)
    (torch.matmul(T, x) * torch.tensor(dy)).sum().backward()
    dx, dT = oracle.mix_bwd(T0, x0, dy)
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dT, T.grad.numpy(), rtol=0, atol=1e-12)


def test_chain_through_the_projection_against_finite_differences():
    """dL/dH for L = <dy, proj(H) x>: the mixing backward's dT fed to the eq (13)
    backward, against central differences of L through the projection."""
    rng = np.random.default_rng(204)
    H = rng.standard_normal((3, 4, 4))
    x = rng.standard_normal((3, 4, 20))
    dy = rng.standard_normal((3, 4, 20))
    T, _, _ = oracle.project(H)
    _, dT = oracle.mix_bwd(T, x, dy)
    dH = oracle.bwd(T, dT)
    h = 1e-5
    fd = np.zeros_like(H)
    for i in range(4):
        for j in range(4):
            Hp, Hm = H.copy(), H.copy()
            Hp[:, i, j] += h
            Hm[:, i, j] -= h
            Lp = (oracle.mix(oracle.project(Hp)[0], x) * dy).sum((1, 2))
            Lm = (oracle.mix(oracle.project(Hm)[0], x) * dy).sum((1, 2))
            fd[:, i, j] = (Lp - Lm) / (2 * h)
    np.testing.assert_allclose(dH, fd, rtol=0, atol=1e-7)


def test_empty_inputs():
    T = np.zeros((0, 4, 4))
    assert oracle.mix(T, np.zeros((0, 4, 8))).shape == (0, 4, 8)
    T1 = np.eye(4)[None]
    assert oracle.mix(T1, np.zeros((1, 4, 0))).shape == (1, 4, 0)
    dx, dT = oracle.mix_bwd(T1, np.zeros((1, 4, 0)), np.zeros((1, 4, 0)))
    np.testing.assert_array_equal(dT, np.zeros((1, 4, 4)))
