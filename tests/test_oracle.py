"""Pins for the float64 oracle (CPU only).

Every expected value here comes from the pages' definitions, closed forms,
hand-worked fixtures under tests/golden/, library routines (scipy, torch
autograd) or brute force -- never from the oracle itself and never from the
HIP path.  A plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand) fails at least one of these tests; see
test_oracle_mutations.py, which plants such slips and checks that they are
caught.

Sources: "Accelerating Birkhoff Projection for Manifold-Constrained
Hyper-Connections" (cited below as [P] with section / equation).
"""
import math
import pathlib
from fractions import Fraction

import numpy as np
import pytest
from scipy.optimize import minimize
from scipy.special import logsumexp, softmax

import oracle
from birkhoff_projection_amd import workloads as W

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def read_golden(name):
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = np.array([float(Fraction(v)) for v in vals])
    return out


def rand_ds(rng, n, terms=6, floor=0.05):
    """Random strictly positive doubly stochastic matrix: a convex combination of
    permutation matrices (Birkhoff-von Neumann) mixed with J/n."""
    w = rng.dirichlet(np.ones(terms))
    P = np.zeros((n, n))
    for k in range(terms):
        P[np.arange(n), rng.permutation(n)] += w[k]
    return (1 - floor) * P + floor * np.ones((n, n)) / n


def marg(T):
    return max(np.abs(T.sum(-1) - 1).max(), np.abs(T.sum(-2) - 1).max())


# ---------------------------------------------------------------- forward ---

def test_golden_n2_projection():
    g = read_golden("n2_projection.txt")
    H = np.log(g["logits_exp"]).reshape(1, 2, 2)
    T, beta, st = oracle.project(H)
    assert st[0] == 0
    np.testing.assert_allclose(T[0].ravel(), g["T"], rtol=0, atol=1e-13)


def test_golden_ds3_fixed_point():
    g = read_golden("ds3_shifted.txt")
    P = g["P"].reshape(3, 3)
    H = np.log(P) + g["row_shift"][:, None] + g["col_shift"][None, :]
    T, beta, st = oracle.project(H[None])
    assert st[0] == 0
    np.testing.assert_allclose(T[0], P, rtol=0, atol=1e-13)
    np.testing.assert_allclose(beta[0], g["beta"], rtol=0, atol=1e-12)
    Tn, bn, it = oracle.newton(H[None])
    assert it[0] >= 0
    np.testing.assert_allclose(Tn[0], P, rtol=0, atol=1e-13)
    np.testing.assert_allclose(bn[0], g["beta"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("sigma", [0.3, 1.0, 3.0, 8.0])
def test_n2_closed_form(sigma):
    """2x2: T11 = T22 = sqrt(r)/(1+sqrt(r)), r = A11 A22 / (A12 A21)  ([P] section 2.2)."""
    rng = np.random.default_rng(11)
    H = sigma * rng.standard_normal((512, 2, 2))
    T, _, st = oracle.project(H)
    assert (st >= 0).all()
    logr = H[:, 0, 0] + H[:, 1, 1] - H[:, 0, 1] - H[:, 1, 0]
    p = 1.0 / (1.0 + np.exp(-logr / 2))          # sqrt(r)/(1+sqrt(r))
    expect = np.stack([p, 1 - p, 1 - p, p], axis=1).reshape(-1, 2, 2)
    np.testing.assert_allclose(T, expect, rtol=0, atol=1e-12)
    Tn, _, it = oracle.newton(H)
    assert (it >= 0).all()
    np.testing.assert_allclose(Tn, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
def test_doubly_stochastic_fixed_point_with_shifts(n):
    """H = log P + a 1^T + 1 b^T with P in B_n maps to P, beta_j = b_n - b_j  ([P] 2.2, eq 4)."""
    rng = np.random.default_rng(100 + n)
    B = 64
    P = np.stack([rand_ds(rng, n) for _ in range(B)])
    a = 3 * rng.standard_normal((B, n))
    b = 3 * rng.standard_normal((B, n))
    H = np.log(P) + a[:, :, None] + b[:, None, :]
    T, beta, st = oracle.project(H)
    assert (st >= 0).all()
    np.testing.assert_allclose(T, P, rtol=0, atol=1e-12)
    np.testing.assert_allclose(beta, b[:, -1:] - b, rtol=0, atol=1e-10)


@pytest.mark.parametrize("n", [3, 4, 8])
def test_rank_one_maps_to_uniform(n):
    """H = a 1^T + 1 b^T (rank-one A) projects to J/n with beta_j = b_n - b_j."""
    rng = np.random.default_rng(200 + n)
    B = 32
    a = 2 * rng.standard_normal((B, n))
    b = 2 * rng.standard_normal((B, n))
    H = a[:, :, None] + b[:, None, :]
    T, beta, st = oracle.project(H)
    assert (st >= 0).all()
    np.testing.assert_allclose(T, np.full_like(T, 1.0 / n), rtol=0, atol=1e-13)
    np.testing.assert_allclose(beta, b[:, -1:] - b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("key", ["pr1", "hard", "train", "n8", "bw"])
def test_marginals_and_log_structure_on_workloads(key):
    """Output lies in B_n ([P] 2.1) and log T - H = alpha 1^T + 1 beta^T ([P] eq 4)."""
    w = W.WORKLOADS[key]
    H = W.decode_f64(W.make_logits(w, B=192))
    T, beta, st = oracle.project(H, sk_cap=w.sk_cap)
    assert (st >= 0).all(), np.unique(st, return_counts=True)
    assert (T > 0).all()
    assert marg(T) <= 2e-13
    X = np.log(T) - H
    # double centering removes alpha_i + beta_j exactly
    Xc = X - X.mean(axis=2, keepdims=True) - X.mean(axis=1, keepdims=True) + X.mean(axis=(1, 2), keepdims=True)
    assert np.abs(Xc).max() <= 1e-9
    # the column part of X is beta (gauge beta_n = 0)
    bcol = X[:, 0, :] - X[:, 0, -1:]
    np.testing.assert_allclose(bcol, beta, rtol=0, atol=1e-9)


def test_equivariance_and_shift_invariance():
    """proj(P A Q) = P proj(A) Q, proj(A^T) = proj(A)^T, and row/column rescaling of A
    (adding u 1^T + 1 v^T to H) leaves T unchanged ([P] 2.2 uniqueness)."""
    rng = np.random.default_rng(7)
    n, B = 4, 64
    H = 2 * rng.standard_normal((B, n, n))
    T, _, _ = oracle.project(H)
    pr, pc = rng.permutation(n), rng.permutation(n)
    T2, _, _ = oracle.project(H[:, pr][:, :, pc])
    np.testing.assert_allclose(T2, T[:, pr][:, :, pc], rtol=0, atol=1e-12)
    T3, _, _ = oracle.project(np.swapaxes(H, 1, 2))
    np.testing.assert_allclose(T3, np.swapaxes(T, 1, 2), rtol=0, atol=1e-12)
    u = 5 * rng.standard_normal((B, n, 1))
    v = 5 * rng.standard_normal((B, 1, n))
    T4, _, _ = oracle.project(H + u + v)
    np.testing.assert_allclose(T4, T, rtol=0, atol=1e-12)


def kl(Pm, A):
    return (Pm * np.log(Pm / A) - Pm + A).sum(axis=(-1, -2))


def test_kl_optimality_against_random_ds():
    """eq (1): KL(T || A) <= KL(P || A) for every P in B_n (brute force over samples)."""
    rng = np.random.default_rng(8)
    n = 4
    for _ in range(16):
        H = 1.5 * rng.standard_normal((n, n))
        A = np.exp(H)
        T, _, _ = oracle.project(H[None])
        k_t = kl(T[0], A)
        Ps = np.stack([rand_ds(rng, n, floor=rng.uniform(0.01, 0.9)) for _ in range(400)])
        assert (kl(Ps, A) >= k_t - 1e-12).all()
        # small moves inside B_n along (E_ij - E_ik - E_lj + E_lk) only increase KL
        for _ in range(50):
            i, l = rng.choice(n, 2, replace=False)
            j, k = rng.choice(n, 2, replace=False)
            Dm = np.zeros((n, n))
            Dm[i, j] = Dm[l, k] = 1
            Dm[i, k] = Dm[l, j] = -1
            for eps in (1e-3, -1e-3):
                Q = T[0] + eps * Dm
                if (Q > 0).all():
                    assert kl(Q, A) > k_t


@pytest.mark.parametrize("n", [3, 4])
def test_primal_problem_with_constrained_solver(n):
    """Solve eq (1) directly as a constrained problem (scipy SLSQP) and compare."""
    rng = np.random.default_rng(20 + n)
    for _ in range(6):
        H = rng.standard_normal((n, n))
        A = np.exp(H)

        def obj(p):
            Pm = p.reshape(n, n)
            return float((Pm * np.log(Pm / A) - Pm + A).sum())

        def jac(p):
            return np.log(p.reshape(n, n) / A).ravel()

        cons = [{"type": "eq", "fun": (lambda p, i=i: p.reshape(n, n)[i].sum() - 1)} for i in range(n)]
        cons += [{"type": "eq", "fun": (lambda p, j=j: p.reshape(n, n)[:, j].sum() - 1)} for j in range(n - 1)]
        r = minimize(obj, np.full(n * n, 1.0 / n), jac=jac, constraints=cons, method="SLSQP",
                     bounds=[(1e-12, None)] * (n * n), options={"ftol": 1e-15, "maxiter": 1000})
        T, _, _ = oracle.project(H[None])
        np.testing.assert_allclose(T[0].ravel(), r.x, rtol=0, atol=2e-6)


@pytest.mark.parametrize("n", [3, 4, 8])
def test_reduced_dual_with_library_minimiser(n):
    """Minimise f(x) = n + sum_i LSE_i(H_i. + beta) - sum_j beta_j, beta = (x, 0)
    ([P] eq 8 with eq 5) by scipy BFGS, recover T by row softmax ([P] 3.1)."""
    rng = np.random.default_rng(30 + n)
    for _ in range(8):
        H = 2 * rng.standard_normal((n, n))

        def f(x):
            beta = np.append(x, 0.0)
            U = H + beta[None, :]
            val = n + logsumexp(U, axis=1).sum() - beta.sum()
            grad = softmax(U, axis=1).sum(axis=0)[:-1] - 1.0
            return val, grad

        r = minimize(f, np.zeros(n - 1), jac=True, method="BFGS", options={"gtol": 1e-13, "maxiter": 10000})
        beta = np.append(r.x, 0.0)
        T_lib = softmax(H + beta[None, :], axis=1)
        T, b_or, _ = oracle.project(H[None])
        # BFGS stalls near 1e-9 in the gradient; any wrong term shows up at 1e-2
        np.testing.assert_allclose(T[0], T_lib, rtol=0, atol=1e-8)
        np.testing.assert_allclose(b_or[0], beta, rtol=0, atol=1e-6)


@pytest.mark.parametrize("n", [3, 4, 8])
def test_first_newton_step_from_the_sweep_start(n):
    """One Newton update (the full step, on mild inputs) from the start x0 = the dual
    after three Sinkhorn sweeps from v = 1, each beta_j += -log c_j + log c_n with c the
    column sums of the row-normalised exp(H + beta): x1 = x0 - H^{-1} g with g and H the
    finite-difference gradient and Hessian of eq (8) at x0."""
    rng = np.random.default_rng(50 + n)
    H = 0.3 * rng.standard_normal((5, n, n))
    _, beta1, _ = oracle.newton(H, 1e-13, 1)
    for q in range(5):
        Hq = H[q]

        def f(x):
            beta = np.append(x, 0.0)
            return n + logsumexp(Hq + beta[None, :], axis=1).sum() - beta.sum()

        beta = np.zeros(n)
        for _ in range(3):
            c = softmax(Hq + beta[None, :], axis=1).sum(axis=0)
            beta = beta - np.log(c) + np.log(c[-1])
        x0 = beta[:-1]
        k, h = n - 1, 1e-4
        E = np.eye(k) * h
        g = np.array([(f(x0 + E[i]) - f(x0 - E[i])) / (2 * h) for i in range(k)])
        Hs = np.array([[(f(x0 + E[i] + E[j]) - f(x0 + E[i] - E[j]) - f(x0 - E[i] + E[j]) + f(x0 - E[i] - E[j]))
                        / (4 * h * h) for j in range(k)] for i in range(k)])
        np.testing.assert_allclose(beta1[q, :-1], x0 - np.linalg.solve(Hs, g), rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("n,sigma", [(3, 1.0), (4, 1.0), (4, 3.0), (5, 2.0), (8, 1.0)])
def test_newton_and_sinkhorn_agree(n, sigma):
    """Two algorithms, one answer: Newton on eq (8) and Sinkhorn-Knopp eq (2)."""
    rng = np.random.default_rng(40 + n)
    H = sigma * rng.standard_normal((128, n, n))
    Ts, bs, sw, cv = oracle.sinkhorn_tol(H, 1e-13, 100_000)
    Tn, bn, it = oracle.newton(H, 1e-13, 500)
    assert cv.all() and (it >= 0).all()
    assert it.max() <= 40
    np.testing.assert_allclose(Tn, Ts, rtol=0, atol=1e-12)
    np.testing.assert_allclose(bn, bs, rtol=0, atol=1e-9)


def test_hard_inputs_are_certified():
    """sigma = 8 inputs: Sinkhorn often hits the cap; Newton + the fixed-point check certifies."""
    rng = np.random.default_rng(9)
    H = 8 * rng.standard_normal((256, 4, 4))
    T, beta, st = oracle.project(H, sk_cap=5000)
    assert (st >= 0).all(), np.unique(st, return_counts=True)
    assert (st == 1).any()        # some matrices genuinely need the Newton reference
    assert marg(T) <= 2e-13


# ------------------------------------------------------- Sinkhorn baseline ---

def test_golden_sk_one_sweep():
    g = read_golden("sk_one_sweep_2x2.txt")
    H = np.log(g["logits_exp"]).reshape(1, 2, 2)
    T = oracle.sinkhorn_k(H, int(g["sweeps"][0]))
    np.testing.assert_allclose(T[0].ravel(), g["T"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("K", [1, 2, 5, 20])
def test_sinkhorn_k_matches_multiplicative_form(K):
    """The log-form sweeps equal eq (2) run in the multiplicative domain (u = 1/(Av), v = 1/(A^T u))."""
    rng = np.random.default_rng(50 + K)
    H = 1.5 * rng.standard_normal((64, 4, 4))
    A = np.exp(H)
    v = np.ones((64, 4))
    for _ in range(K):
        u = 1.0 / np.einsum("bij,bj->bi", A, v)
        v = 1.0 / np.einsum("bij,bi->bj", A, u)
    expect = u[:, :, None] * A * v[:, None, :]
    T = oracle.sinkhorn_k(H, K)
    np.testing.assert_allclose(T, expect, rtol=1e-12, atol=0)
    np.testing.assert_allclose(T.sum(axis=1), 1.0, rtol=0, atol=1e-14)   # columns exact after a sweep


def test_sinkhorn_k_converges_to_projection():
    rng = np.random.default_rng(60)
    H = rng.standard_normal((32, 4, 4))
    T, _, _ = oracle.project(H)
    np.testing.assert_allclose(oracle.sinkhorn_k(H, 3000), T, rtol=0, atol=1e-13)


# --------------------------------------------------------------- backward ---

def test_golden_n2_backward():
    g = read_golden("n2_projection.txt")
    H = np.log(g["logits_exp"]).reshape(1, 2, 2)
    T, _, _ = oracle.project(H)
    dH = oracle.bwd(T, g["G"].reshape(1, 2, 2))
    np.testing.assert_allclose(dH[0].ravel(), g["dH"], rtol=0, atol=1e-14)


def test_n2_backward_closed_form():
    """p = sigmoid((H11+H22-H12-H21)/2):  dH = s p(1-p)/2 [[1,-1],[-1,1]], s = G11+G22-G12-G21."""
    rng = np.random.default_rng(12)
    H = 2 * rng.standard_normal((256, 2, 2))
    G = rng.standard_normal((256, 2, 2))
    T, _, _ = oracle.project(H)
    dH = oracle.bwd(T, G)
    p = T[:, 0, 0]
    s = G[:, 0, 0] + G[:, 1, 1] - G[:, 0, 1] - G[:, 1, 0]
    k = s * p * (1 - p) / 2
    expect = np.stack([k, -k, -k, k], axis=1).reshape(-1, 2, 2)
    np.testing.assert_allclose(dH, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,sigma", [(3, 1.0), (4, 1.0), (4, 3.0), (8, 1.0)])
def test_backward_central_differences(n, sigma):
    """eq (13) + sign flip against central differences of <G, proj(exp(H))>."""
    rng = np.random.default_rng(70 + n)
    B = 6
    H = sigma * rng.standard_normal((B, n, n))
    G = rng.standard_normal((B, n, n))
    T, _, _ = oracle.project(H)
    dH = oracle.bwd(T, G)
    h = 1e-5
    fd = np.empty_like(dH)
    for k in range(n * n):
        E = np.zeros((n, n))
        E.flat[k] = h
        Tp, _, _ = oracle.project(H + E)
        Tm, _, _ = oracle.project(H - E)
        fd[:, k // n, k % n] = ((G * Tp).sum(axis=(1, 2)) - (G * Tm).sum(axis=(1, 2))) / (2 * h)
    np.testing.assert_allclose(dH, fd, rtol=0, atol=1e-7)


def test_backward_invariants():
    """dH has zero row and column sums (T is invariant to row/column shifts of H), and
    G = u 1^T + 1 v^T gives dH = 0 (<G, T> is then constant on B_n)."""
    rng = np.random.default_rng(13)
    for n in (3, 4, 8):
        H = 2 * rng.standard_normal((64, n, n))
        T, _, _ = oracle.project(H)
        G = rng.standard_normal((64, n, n))
        dH = oracle.bwd(T, G)
        scale = np.abs(dH).max()
        # T meets the marginals to 1e-13, so the invariants hold to that order
        assert np.abs(dH.sum(axis=1)).max() <= 1e-12 * max(1.0, scale)
        assert np.abs(dH.sum(axis=2)).max() <= 1e-12 * max(1.0, scale)
        G0 = rng.standard_normal((64, n, 1)) + rng.standard_normal((64, 1, n))
        assert np.abs(oracle.bwd(T, G0)).max() <= 1e-12


def test_backward_matches_unrolled_autograd():
    """Differentiate 2000 unrolled log-domain Sinkhorn sweeps with torch float64 autograd
    (the approach the implicit backward replaces) and compare."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    for n in (4, 8):
        H0 = rng.standard_normal((8, n, n))
        G = rng.standard_normal((8, n, n))
        H = torch.tensor(H0, dtype=torch.float64, requires_grad=True)
        beta = torch.zeros(8, 1, n, dtype=torch.float64)
        for _ in range(2000):
            alpha = -torch.logsumexp(H + beta, dim=2, keepdim=True)
            beta = -torch.logsumexp(H + alpha, dim=1, keepdim=True)
        T = torch.exp(H + alpha + beta)
        (T * torch.tensor(G)).sum().backward()
        Tref, _, _ = oracle.project(H0)
        dH = oracle.bwd(Tref, G)
        np.testing.assert_allclose(dH, H.grad.numpy(), rtol=0, atol=1e-10)


# ------------------------------------------------------------ arguments ---

def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.project(np.zeros((1, 1, 1)))
    with pytest.raises(ValueError):
        oracle.project(np.zeros((1, 17, 17)))
    T, _, st = oracle.project(np.zeros((0, 4, 4)))
    assert T.shape == (0, 4, 4)
