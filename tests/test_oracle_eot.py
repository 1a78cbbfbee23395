"""Pins for the float64 oracle's general small entropic OT (CPU only).

The general problem of [P] section 2.3 (eq 3): a cost M (n x m), marginals
a > 0 and b > 0 with equal sums, and eta > 0.  As in test_oracle.py, every
expected value comes from a closed form, a hand-worked fixture under
tests/golden/, an invariant the mathematics fixes, a library routine (scipy,
torch autograd) or the Birkhoff special case, whose oracle is pinned on its
own -- never from these functions themselves.  test_oracle_mutations.py plants
slips in this part of the oracle too and checks that they are caught here.

Sources: "Accelerating Birkhoff Projection for Manifold-Constrained
Hyper-Connections" ([P]), section 2.3 (eqs 3-7), section 3.1 (eqs 8-9),
section 4.1 (eq 13).
"""
import pathlib
from fractions import Fraction

import numpy as np
import pytest
from scipy.optimize import minimize
from scipy.special import logsumexp, softmax

import oracle

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"

SHAPES = [(1, 2), (1, 5), (2, 2), (2, 3), (3, 2), (3, 5), (5, 3), (4, 4), (2, 8), (8, 2), (7, 8), (8, 8), (6, 7)]


def read_golden(name):
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = np.array([float(Fraction(v)) for v in vals])
    return out


def problem(rng, B, n, m, sigma=1.0, total=1.0):
    """Random costs and strictly positive marginals with equal sums."""
    M = sigma * rng.standard_normal((B, n, m))
    a = rng.uniform(0.2, 1.0, (B, n))
    b = rng.uniform(0.2, 1.0, (B, m))
    a *= total / a.sum(1, keepdims=True)
    b *= total / b.sum(1, keepdims=True)
    return M, a, b


def marg_err(T, a, b):
    return max(np.abs(T.sum(-1) - a).max(), np.abs(T.sum(-2) - b).max())


# ---------------------------------------------------------------- forward ---

def test_golden_2x2_plan():
    """Hand-worked 2 x 2 case (tests/golden/eot_2x2.txt): the plan with the given
    marginals whose cross ratio T11 T22 / (T12 T21) is exp(-(M11+M22-M12-M21)/eta)."""
    g = read_golden("eot_2x2.txt")
    eta = float(g["eta"][0])
    M = np.array([[0.0, 0.0], [0.0, -eta * np.log(float(g["cross_ratio"][0]))]])
    T, beta, st = oracle.eot_project(M, g["a"], g["b"], eta)
    assert st[0] == 0
    np.testing.assert_allclose(T[0].ravel(), g["T"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("eta", [0.25, 1.0, 4.0])
def test_2x2_closed_form(eta):
    """n = m = 2: T = [[t, a1 - t], [b1 - t, a2 - b1 + t]] with the cross ratio
    kappa = exp(-(M11 + M22 - M12 - M21) / eta) (eq 4), i.e. t solves
    (1 - kappa) t^2 + (a2 - b1 + kappa (a1 + b1)) t - kappa a1 b1 = 0."""
    rng = np.random.default_rng(101)
    M, a, b = problem(rng, 64, 2, 2, sigma=1.5)
    T, beta, st = oracle.eot_project(M, a, b, eta)
    assert (st == 0).all()
    for q in range(64):
        kap = np.exp(-(M[q, 0, 0] + M[q, 1, 1] - M[q, 0, 1] - M[q, 1, 0]) / eta)
        a1, a2 = a[q]
        b1 = b[q, 0]
        roots = np.roots([1 - kap, a2 - b1 + kap * (a1 + b1), -kap * a1 * b1])
        lo, hi = max(0.0, b1 - a2), min(a1, b1)
        t = [r.real for r in roots if abs(r.imag) < 1e-12 and lo < r.real < hi]
        assert len(t) == 1
        np.testing.assert_allclose(T[q, 0, 0], t[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,m", SHAPES)
def test_separable_cost_gives_product_plan(n, m):
    """M_ij = u_i + v_j: the plan is a b^T / sum(a) (it factorises as eq 4 demands and
    meets both marginals), and beta_j - beta_m = eta log(b_j / b_m) + v_j - v_m."""
    rng = np.random.default_rng(102 + 10 * n + m)
    B, eta = 16, 0.7
    _, a, b = problem(rng, B, n, m, total=2.5)
    u = rng.standard_normal((B, n, 1))
    v = rng.standard_normal((B, 1, m))
    M = u + v
    for T, beta in (oracle.eot_project(M, a, b, eta)[:2], oracle.eot_newton(M, a, b, eta)[:2],
                    oracle.eot_sinkhorn_tol(M, a, b, eta)[:2]):
        np.testing.assert_allclose(T, a[:, :, None] * b[:, None, :] / 2.5, rtol=0, atol=1e-13)
        ref = eta * np.log(b / b[:, -1:]) + v[:, 0, :] - v[:, 0, -1:]
        np.testing.assert_allclose(beta, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("n,m", SHAPES)
@pytest.mark.parametrize("eta", [0.3, 1.0, 3.0])
def test_certificate_on_random_problems(n, m, eta):
    """Optimality certificate of eq (4): the plan meets both marginals and
    eta log T + M is a row term plus a column term (alpha_i + beta_j), whose column
    part is the reported beta in the gauge beta_m = 0.  The two conditions fix the
    plan uniquely."""
    rng = np.random.default_rng(103 + 10 * n + m)
    M, a, b = problem(rng, 32, n, m, sigma=2.0)
    T, beta, st = oracle.eot_project(M, a, b, eta)
    assert (st >= 0).all()
    assert marg_err(T, a, b) <= 1e-12
    R = eta * np.log(T) + M
    dc = R - R.mean(2, keepdims=True) - R.mean(1, keepdims=True) + R.mean((1, 2), keepdims=True)
    assert np.abs(dc).max() <= 1e-10
    col = (R - R[:, :, -1:]).mean(1)
    np.testing.assert_allclose(beta, col, rtol=0, atol=1e-10)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_birkhoff_special_case(n):
    """a = b = 1, eta = 1, M = -H is the Birkhoff projection ([P] end of section 2.3),
    whose oracle is pinned separately in test_oracle.py."""
    rng = np.random.default_rng(104 + n)
    H = 1.5 * rng.standard_normal((32, n, n))
    T0, b0, _ = oracle.project(H)
    T, beta, st = oracle.eot_project(-H, np.ones(n), np.ones(n), 1.0)
    assert (st >= 0).all()
    np.testing.assert_allclose(T, T0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(beta, b0, rtol=0, atol=1e-11)


def test_eta_scaling_transpose_and_homogeneity():
    """Three symmetries of eq (3): the plan for (M, eta) equals the plan for (M/eta, 1)
    with beta scaled by eta; the plan for (M^T, b, a) is the transpose; and scaling
    both marginals by lam scales the plan by lam and leaves beta unchanged."""
    rng = np.random.default_rng(105)
    for n, m in ((3, 5), (5, 3), (4, 4), (2, 7)):
        M, a, b = problem(rng, 24, n, m, sigma=2.0)
        eta = 0.37
        T, beta, _ = oracle.eot_project(M, a, b, eta)
        T1, beta1, _ = oracle.eot_project(M / eta, a, b, 1.0)
        # each solve meets the marginals to 1e-13, so two solves agree to a few 1e-13
        np.testing.assert_allclose(T, T1, rtol=0, atol=5e-13)
        np.testing.assert_allclose(beta, eta * beta1, rtol=0, atol=1e-11)
        Tt, _, _ = oracle.eot_project(np.swapaxes(M, 1, 2), b, a, eta)
        np.testing.assert_allclose(Tt, np.swapaxes(T, 1, 2), rtol=0, atol=5e-13)
        Tl, betal, _ = oracle.eot_project(M, 3.0 * a, 3.0 * b, eta)
        np.testing.assert_allclose(Tl, 3.0 * T, rtol=0, atol=1.5e-12)
        np.testing.assert_allclose(betal, beta, rtol=0, atol=1e-10)


@pytest.mark.parametrize("n,m", [(2, 3), (3, 4), (4, 3)])
def test_primal_problem_with_constrained_solver(n, m):
    """Solve eq (3) directly: min <T, M> + eta sum T (log T - 1) subject to T 1 = a and
    T^T 1 = b (scipy SLSQP)."""
    rng = np.random.default_rng(106 + n * m)
    eta = 0.6
    for _ in range(5):
        M, a, b = problem(rng, 1, n, m)
        Mq, aq, bq = M[0], a[0], b[0]

        def obj(p):
            P = p.reshape(n, m)
            return float((P * Mq).sum() + eta * (P * (np.log(P) - 1)).sum())

        def jac(p):
            return (Mq + eta * np.log(p.reshape(n, m))).ravel()

        cons = [{"type": "eq", "fun": (lambda p, i=i: p.reshape(n, m)[i].sum() - aq[i])} for i in range(n)]
        cons += [{"type": "eq", "fun": (lambda p, j=j: p.reshape(n, m)[:, j].sum() - bq[j])} for j in range(m - 1)]
        r = minimize(obj, np.outer(aq, bq).ravel(), jac=jac, constraints=cons, method="SLSQP",
                     bounds=[(1e-12, None)] * (n * m), options={"ftol": 1e-15, "maxiter": 2000})
        T, _, _ = oracle.eot_project(M, a, b, eta)
        np.testing.assert_allclose(T[0].ravel(), r.x, rtol=0, atol=2e-6)


@pytest.mark.parametrize("n,m", [(3, 4), (4, 3), (5, 6), (8, 8)])
def test_reduced_dual_with_library_minimiser(n, m):
    """Minimise eq (8), f(x) = eta 1^T a - alpha*(beta)^T a - beta^T b with
    beta = (x, 0) and alpha* from eq (5), by scipy BFGS on finite differences, then
    recover the plan from eq (4)."""
    rng = np.random.default_rng(107 + n * m)
    eta = 0.8
    for _ in range(4):
        M, a, b = problem(rng, 1, n, m, sigma=1.5)
        Mq, aq, bq = M[0], a[0], b[0]

        def f(x):
            beta = np.append(x, 0.0)
            alpha = eta * np.log(aq) - eta * logsumexp((beta[None, :] - Mq) / eta, axis=1)
            return eta * aq.sum() - alpha @ aq - beta @ bq

        r = minimize(f, np.zeros(m - 1), method="BFGS", options={"gtol": 1e-11, "maxiter": 20000})
        beta = np.append(r.x, 0.0)
        alpha = eta * np.log(aq) - eta * logsumexp((beta[None, :] - Mq) / eta, axis=1)
        T_lib = np.exp((alpha[:, None] + beta[None, :] - Mq) / eta)
        T, b_or, _ = oracle.eot_project(M, a, b, eta)
        np.testing.assert_allclose(T[0], T_lib, rtol=0, atol=1e-6)
        np.testing.assert_allclose(b_or[0], beta, rtol=0, atol=1e-5)


@pytest.mark.parametrize("eta", [0.3, 3.0])
def test_first_newton_step_matches_finite_difference_newton(eta):
    """One Newton update from the start on a mild problem (the full step is taken):
    x1 = x0 - H^{-1} g, with g and H the finite-difference gradient and Hessian of eq (8)
    at x0, the dual after three Sinkhorn sweeps (eqs 5-6) from beta = eta log(b / b_m)."""
    rng = np.random.default_rng(108)
    n, m = 4, 5
    M, a, b = problem(rng, 6, n, m, sigma=0.3 * eta)
    _, beta1, _ = oracle.eot_newton(M, a, b, eta, tol=1e-13, max_iter=1)
    for q in range(6):
        Mq, aq, bq = M[q], a[q], b[q]

        def f(x):
            beta = np.append(x, 0.0)
            alpha = eta * np.log(aq) - eta * logsumexp((beta[None, :] - Mq) / eta, axis=1)
            return eta * aq.sum() - alpha @ aq - beta @ bq

        k, h = m - 1, 1e-4 * eta
        b_sweep = eta * (np.log(bq) - np.log(bq[-1]))
        for _ in range(3):
            a_sweep = eta * np.log(aq) - eta * logsumexp((b_sweep[None, :] - Mq) / eta, axis=1)   # eq (5)
            b_sweep = eta * np.log(bq) - eta * logsumexp((a_sweep[:, None] - Mq) / eta, axis=0)  # eq (6)
        x0 = b_sweep[:-1] - b_sweep[-1]
        E = np.eye(k) * h
        g = np.array([(f(x0 + E[i]) - f(x0 - E[i])) / (2 * h) for i in range(k)])
        Hs = np.array([[(f(x0 + E[i] + E[j]) - f(x0 + E[i] - E[j]) - f(x0 - E[i] + E[j]) + f(x0 - E[i] - E[j]))
                        / (4 * h * h) for j in range(k)] for i in range(k)])
        x1 = x0 - np.linalg.solve(Hs, g)
        np.testing.assert_allclose(beta1[q, :-1], x1, rtol=1e-5, atol=1e-7 * eta)


def test_constant_cost_needs_no_update():
    """A constant cost has the plan a b^T / sum(b); the start (sweeps from
    eta log(b / b_m)) is already optimal, so Newton stops before its first update."""
    rng = np.random.default_rng(115)
    M, a, b = problem(rng, 8, 3, 6)
    M[:] = 0.7
    T, beta, it = oracle.eot_newton(M, a, b, 0.4, tol=1e-12)
    assert (it == 0).all()
    np.testing.assert_allclose(T, a[:, :, None] * b[:, None, :], rtol=0, atol=1e-14)


@pytest.mark.parametrize("n,m", [(3, 5), (5, 3), (4, 4), (8, 8), (1, 4)])
@pytest.mark.parametrize("eta", [0.3, 1.0, 3.0])
def test_newton_and_sinkhorn_agree(n, m, eta):
    """Newton on eq (8) and Sinkhorn-Knopp (eq 7) give one plan; Newton converges in
    few updates (its line search and fallback only steer, so a mis-scaled step shows
    up in the count)."""
    rng = np.random.default_rng(109 + n * m)
    M, a, b = problem(rng, 96, n, m, sigma=1.0 * eta)
    Ts, bs, sw, cv = oracle.eot_sinkhorn_tol(M, a, b, eta, 1e-13, 100_000)
    Tn, bn, it = oracle.eot_newton(M, a, b, eta, 1e-13, 500)
    assert cv.all() and (it >= 0).all()
    assert it.max() <= 12
    np.testing.assert_allclose(Tn, Ts, rtol=0, atol=1e-12)
    np.testing.assert_allclose(bn, bs, rtol=0, atol=1e-9 * eta)


def test_sinkhorn_one_sweep_by_hand():
    """One sweep of eq (7) from beta = 0, multiplicatively: u = a / (K 1), v = b / (K^T u)
    with K = exp(-M / eta); after it the column marginals are exact."""
    rng = np.random.default_rng(110)
    M, a, b = problem(rng, 8, 3, 4)
    eta = 0.9
    T, _, sw, _ = oracle.eot_sinkhorn_tol(M, a, b, eta, tol=0.0, cap=1)
    assert (sw == 1).all()
    K = np.exp(-M / eta)
    u = a / K.sum(2)
    v = b / np.einsum("bij,bi->bj", K, u)
    np.testing.assert_allclose(T, u[:, :, None] * K * v[:, None, :], rtol=1e-14, atol=0)


# --------------------------------------------------------------- backward ---

@pytest.mark.parametrize("n,m", [(3, 5), (5, 3), (4, 4), (2, 2), (1, 3)])
@pytest.mark.parametrize("eta", [0.4, 2.0])
def test_backward_central_differences(n, m, eta):
    """eq (13) against central differences of <G, T*(M)>, with T*(M) from the
    (separately pinned) forward."""
    rng = np.random.default_rng(111 + n * m)
    M, a, b = problem(rng, 4, n, m, sigma=1.0)
    G = rng.standard_normal((4, n, m))
    T, _, _ = oracle.eot_project(M, a, b, eta)
    D = oracle.eot_bwd(T, G, a, b, eta)
    h = 1e-5
    fd = np.zeros_like(M)
    for i in range(n):
        for j in range(m):
            Mp, Mm = M.copy(), M.copy()
            Mp[:, i, j] += h
            Mm[:, i, j] -= h
            Tp, _, _ = oracle.eot_project(Mp, a, b, eta)
            Tm, _, _ = oracle.eot_project(Mm, a, b, eta)
            fd[:, i, j] = ((Tp - Tm) * G).sum((1, 2)) / (2 * h)
    np.testing.assert_allclose(D, fd, rtol=0, atol=2e-7)


def test_backward_invariants():
    """The plan is unchanged by adding u 1^T + 1 v^T to M, so D has zero row and column
    sums; and G = u 1^T + 1 v^T makes <G, T*> = u^T a + v^T b constant, so D = 0."""
    rng = np.random.default_rng(112)
    for n, m in ((3, 5), (5, 3), (8, 8)):
        M, a, b = problem(rng, 32, n, m, sigma=2.0)
        eta = 0.6
        T, _, _ = oracle.eot_project(M, a, b, eta)
        G = rng.standard_normal((32, n, m))
        D = oracle.eot_bwd(T, G, a, b, eta)
        scale = max(1.0, np.abs(D).max())
        assert np.abs(D.sum(1)).max() <= 1e-11 * scale
        assert np.abs(D.sum(2)).max() <= 1e-11 * scale
        G0 = rng.standard_normal((32, n, 1)) + rng.standard_normal((32, 1, m))
        assert np.abs(oracle.eot_bwd(T, G0, a, b, eta)).max() <= 1e-11


def test_backward_birkhoff_special_case():
    """a = b = 1, eta = 1, M = -H: D = dl/dM = -dl/dH, the Birkhoff backward pinned in
    test_oracle.py."""
    rng = np.random.default_rng(113)
    for n in (3, 4, 8):
        H = rng.standard_normal((16, n, n))
        T, _, _ = oracle.project(H)
        G = rng.standard_normal((16, n, n))
        D = oracle.eot_bwd(T, G, np.ones(n), np.ones(n), 1.0)
        np.testing.assert_allclose(D, -oracle.bwd(T, G), rtol=0, atol=1e-13)


def test_backward_matches_unrolled_autograd():
    """Differentiate 3000 unrolled log-domain sweeps of eq (7) (general a, b, eta) with
    torch float64 autograd and compare."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(114)
    for n, m in ((3, 5), (6, 4)):
        M0, a0, b0 = problem(rng, 6, n, m, sigma=1.0)
        G = rng.standard_normal((6, n, m))
        eta = 0.7
        M = torch.tensor(M0, requires_grad=True)
        la = torch.log(torch.tensor(a0))[:, :, None]
        lb = torch.log(torch.tensor(b0))[:, None, :]
        beta = torch.zeros(6, 1, m, dtype=torch.float64)
        for _ in range(3000):
            alpha = eta * la - eta * torch.logsumexp((beta - M) / eta, dim=2, keepdim=True)
            beta = eta * lb - eta * torch.logsumexp((alpha - M) / eta, dim=1, keepdim=True)
        T = torch.exp((alpha + beta - M) / eta)
        (T * torch.tensor(G)).sum().backward()
        Tref, _, _ = oracle.eot_project(M0, a0, b0, eta)
        D = oracle.eot_bwd(Tref, G, a0, b0, eta)
        np.testing.assert_allclose(D, M.grad.numpy(), rtol=0, atol=1e-10)


# ------------------------------------------------------------ arguments ---

def test_rejects_bad_arguments():
    a, b = np.ones(3) / 3, np.ones(4) / 4
    with pytest.raises(ValueError):
        oracle.eot_project(np.zeros((1, 3, 4)), a, b, 0.0)
    with pytest.raises(ValueError):
        oracle.eot_project(np.zeros((1, 3, 1)), a, np.ones(1), 1.0)
    with pytest.raises(ValueError):
        oracle.eot_project(np.zeros((1, 17, 4)), np.ones(17) / 17, b, 1.0)
    T, beta, st = oracle.eot_project(np.zeros((0, 3, 4)), a, b, 1.0)
    assert T.shape == (0, 3, 4) and beta.shape == (0, 4)
