"""GPU parity for the general small entropic OT (birkhoff_eot_fwd / birkhoff_eot_bwd,
through the C ABI) against the float64 oracle on the same seeded inputs.  Needs an
MI355X; run with -m gpu.

Gates, those of the Birkhoff path scaled by the plan's total mass s = sum(a)
(every workload here has s = 1 exactly):
  forward   max |T - T_ref| <= 1e-5 s over every entry;
  residual  max(|T 1 - a|, |T^T 1 - b|) of the GPU's T, summed in float64, <= 1e-5 s;
  dual      the plan rebuilt in float64 from (cost, a, dual) as
            T_ij = a_i Softmax_j((beta_j - M_ij) / eta) matches the GPU's T to 1e-5 s;
  backward  per problem max|D - D_ref| / max(max|D_ref|, 0.04 max|G o T_ref| / eta) <= 1e-4.
            D_ij = T_ij (nu_i - (S w)_i + w_j - G_ij) / eta sums terms of D's natural
            size |G o T| / eta that can cancel, and w comes from an (m-1)-dimensional
            solve; fp32 leaves an absolute error of some tens of ulps of that size
            (up to 1.1e-6 of it measured over every shape), so where the exact gradient
            is small or vanishes (n = 1: the only plan is b^T, whatever the cost) the
            gate falls back to 4e-6 |G o T| / eta.
"""
import numpy as np
import pytest

import oracle
from birkhoff_projection_amd import workloads as W

torch = pytest.importorskip("torch")
import birkhoff_projection_amd as bp  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

FWD_TOL = 1e-5
RES_TOL = 1e-5
BWD_TOL = 1e-4
SHAPES = [(n, m) for n in range(1, 9) for m in range(2, 9)]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def f64(t):
    return t.cpu().numpy().astype(np.float64)


def workload(n, m, eta=0.5, sigma=1.0, shared=False, seed=60):
    return W.EotWorkload(key="eot_%dx%d" % (n, m), title="test", B=0, n=n, m=m, eta=eta,
                         cost=("normal", sigma), marginals=("dyadic", 0.5, 1.5), upstream=("normal", 1.0),
                         seed=seed, shared=shared)


def residual(T, a, b):
    return np.maximum(np.abs(T.sum(-1) - a).max(-1), np.abs(T.sum(-2) - b).max(-1))


def rebuilt(M, a, dual, eta):
    U = (dual[:, None, :] - M) / eta
    U = U - U.max(axis=2, keepdims=True)
    E = np.exp(U)
    return a[:, :, None] * E / E.sum(axis=2, keepdims=True)


def check_forward(M, a, b, eta, T, dual, iters=None, tol=1e-6):
    """All forward gates against the oracle; returns the oracle's plan."""
    B, n, m = M.shape
    a2 = np.broadcast_to(a, (B, n)).astype(np.float64)
    b2 = np.broadcast_to(b, (B, m)).astype(np.float64)
    T_ref, _, st = oracle.eot_project(M.astype(np.float64), a2, b2, eta)
    assert (st >= 0).all()
    Tg, dg = f64(T), f64(dual)
    err = np.abs(Tg - T_ref).max()
    assert err <= FWD_TOL, "max|T - T_ref| = %.3e" % err
    assert residual(Tg, a2, b2).max() <= RES_TOL
    assert np.abs(rebuilt(M.astype(np.float64), a2, dg, eta) - Tg).max() <= FWD_TOL
    assert np.all(dg[:, -1] == 0.0)
    if iters is not None:
        it = iters.cpu().numpy()
        assert (it >= 0).all(), "unconverged problems: %d" % (it < 0).sum()
    return T_ref


def check_backward(D, D_ref, G, T_ref, eta):
    Dg = f64(D)
    natural = np.abs(G * T_ref).max(axis=(1, 2)) / eta
    scale = np.maximum(np.abs(D_ref).max(axis=(1, 2)), 0.04 * natural)
    rel = np.abs(Dg - D_ref).max(axis=(1, 2)) / np.where(scale > 0, scale, 1.0)
    assert rel.max() <= BWD_TOL, "worst relative backward error %.3e" % rel.max()


# ---------------------------------------------------------------- forward ---

@pytest.mark.parametrize("n,m", SHAPES)
def test_forward_every_shape(n, m):
    """Every supported shape at B = 300: full waves and a ragged last wave."""
    w = workload(n, m)
    M, a, b = W.make_eot(w, B=300)
    print("eot fwd n=%d m=%d B=300" % (n, m), flush=True)
    T, dual, iters = bp.eot_plan(dev(M), dev(a), dev(b), w.eta, with_iters=True)
    torch.cuda.synchronize()
    check_forward(M, a, b, w.eta, T, dual, iters)


@pytest.mark.parametrize("n,m", [(1, 2), (3, 5), (4, 6), (8, 3), (8, 8)])
@pytest.mark.parametrize("B", [1, 63, 64, 65, 255, 257, 1000])
def test_forward_ragged_batches(n, m, B):
    w = workload(n, m, seed=61)
    M, a, b = W.make_eot(w, B=B)
    print("eot ragged n=%d m=%d B=%d" % (n, m, B), flush=True)
    T, dual = bp.eot_plan(dev(M), dev(a), dev(b), w.eta)
    torch.cuda.synchronize()
    check_forward(M, a, b, w.eta, T, dual)


@pytest.mark.parametrize("eta", [0.125, 0.25, 2.0, 8.0])
def test_forward_eta_range(eta):
    """Small eta sharpens the plans (cost / eta up to ~30): more Newton updates,
    same gates.  At eta = 1/8 the step rule crawls on a few problems (the
    float64 oracle's Newton, run with the same rule, needs up to ~150 updates
    on 20,000 such problems), so the cap is raised to 200."""
    w = workload(4, 6, eta=eta, seed=62)
    M, a, b = W.make_eot(w, B=2048)
    print("eot eta=%g" % eta, flush=True)
    T, dual, iters = bp.eot_plan(dev(M), dev(a), dev(b), eta, max_iter=200, with_iters=True)
    torch.cuda.synchronize()
    check_forward(M, a, b, eta, T, dual, iters)


def test_shared_marginals_equal_per_problem_copies():
    """One (a, b) pair for the batch gives bit-identical results to the same pair
    repeated per problem."""
    w = workload(5, 7, shared=True, seed=63)
    M, a, b = W.make_eot(w, B=777)
    T1, d1, i1 = bp.eot_plan(dev(M), dev(a), dev(b), w.eta, with_iters=True)
    A = np.ascontiguousarray(np.broadcast_to(a, (777, 5)))
    Bm = np.ascontiguousarray(np.broadcast_to(b, (777, 7)))
    T2, d2, i2 = bp.eot_plan(dev(M), dev(A), dev(Bm), w.eta, with_iters=True)
    torch.cuda.synchronize()
    assert torch.equal(T1, T2) and torch.equal(d1, d2) and torch.equal(i1, i2)
    check_forward(M, a, b, w.eta, T1, d1, i1)


def test_iteration_counts_do_not_change_results():
    w = workload(4, 6, seed=64)
    M, a, b = W.make_eot(w, B=4096)
    T1, d1 = bp.eot_plan(dev(M), dev(a), dev(b), w.eta)
    T2, d2, it = bp.eot_plan(dev(M), dev(a), dev(b), w.eta, with_iters=True)
    torch.cuda.synchronize()
    assert torch.equal(T1, T2) and torch.equal(d1, d2)
    it = it.cpu().numpy()
    assert (it >= 0).all() and it.max() <= 20


def test_birkhoff_special_case():
    """a = b = 1, eta = 1, cost = -H on the 4x4 Birkhoff inputs: the Birkhoff projection
    and its backward (dL/dM = -dL/dH)."""
    wb = W.WORKLOADS["pr1"]
    H = W.make_logits(wb, B=4096)
    G = W.make_upstream(wb, B=4096)
    ones = dev(np.ones(4, dtype=np.float32))
    T, dual = bp.eot_plan(dev(-H), ones, ones, 1.0)
    D = bp.eot_plan_bwd(T, dev(G), ones, 1.0)
    torch.cuda.synchronize()
    T_ref, _, st = oracle.project(H.astype(np.float64))
    assert (st >= 0).all()
    assert np.abs(f64(T) - T_ref).max() <= FWD_TOL
    check_backward(D, -oracle.bwd(T_ref, G.astype(np.float64)), G.astype(np.float64), T_ref, 1.0)


def test_single_row_and_separable_costs_have_closed_forms():
    """n = 1: the only plan is T = b^T (a_1 = 1).  Separable costs M_ij = u_i + v_j:
    the plan is a b^T."""
    rng = np.random.default_rng(65)
    w1 = workload(1, 6, seed=65)
    M, a, b = W.make_eot(w1, B=500)
    T, dual = bp.eot_plan(dev(M), dev(a), dev(b), w1.eta)
    torch.cuda.synchronize()
    assert np.abs(f64(T)[:, 0, :] - b.astype(np.float64)).max() <= FWD_TOL
    w2 = workload(5, 4, seed=66)
    _, a, b = W.make_eot(w2, B=500)
    M = (rng.standard_normal((500, 5, 1)) + rng.standard_normal((500, 1, 4))).astype(np.float32)
    T, dual = bp.eot_plan(dev(M), dev(a), dev(b), w2.eta)
    torch.cuda.synchronize()
    ab = a.astype(np.float64)[:, :, None] * b.astype(np.float64)[:, None, :]
    assert np.abs(f64(T) - ab).max() <= FWD_TOL


def test_empty_batch_is_a_no_op():
    M = torch.empty((0, 3, 5), dtype=torch.float32, device=DEV)
    a = torch.empty((0, 3), dtype=torch.float32, device=DEV)
    b = torch.empty((0, 5), dtype=torch.float32, device=DEV)
    T, dual = bp.eot_plan(M, a, b, 0.5)
    D = bp.eot_plan_bwd(T, torch.empty_like(T), a, 0.5)
    torch.cuda.synchronize()
    assert T.shape == (0, 3, 5) and dual.shape == (0, 5) and D.shape == (0, 3, 5)


# --------------------------------------------------------------- backward ---

@pytest.mark.parametrize("n,m", SHAPES)
def test_backward_every_shape_at_reference_plans(n, m):
    """eq (13) from the oracle's plan (rounded to fp32) against the oracle's
    backward at the same plan."""
    w = workload(n, m, seed=67)
    M, a, b = W.make_eot(w, B=300)
    G = W.make_eot_upstream(w, B=300)
    T_ref, _, _ = oracle.eot_project(M.astype(np.float64), a.astype(np.float64), b.astype(np.float64), w.eta)
    T32 = T_ref.astype(np.float32)
    print("eot bwd n=%d m=%d" % (n, m), flush=True)
    D = bp.eot_plan_bwd(dev(T32), dev(G), dev(a), w.eta)
    torch.cuda.synchronize()
    D_ref = oracle.eot_bwd(T32.astype(np.float64), G.astype(np.float64), a.astype(np.float64),
                           b.astype(np.float64), w.eta)
    check_backward(D, D_ref, G.astype(np.float64), T32.astype(np.float64), w.eta)


@pytest.mark.parametrize("n,m", [(2, 3), (4, 6), (6, 4), (8, 8)])
def test_forward_then_backward_chain(n, m):
    """The GPU forward's plan fed to the GPU backward, against the oracle's chain."""
    w = workload(n, m, seed=68)
    M, a, b = W.make_eot(w, B=2000)
    G = W.make_eot_upstream(w, B=2000)
    T, _ = bp.eot_plan(dev(M), dev(a), dev(b), w.eta)
    D = bp.eot_plan_bwd(T, dev(G), dev(a), w.eta)
    torch.cuda.synchronize()
    T_ref, _, _ = oracle.eot_project(M.astype(np.float64), a.astype(np.float64), b.astype(np.float64), w.eta)
    check_backward(D, oracle.eot_bwd(T_ref, G.astype(np.float64), a.astype(np.float64),
                                     b.astype(np.float64), w.eta), G.astype(np.float64), T_ref, w.eta)


def test_autograd_function():
    w = workload(3, 5, seed=69)
    M, a, b = W.make_eot(w, B=512)
    G = W.make_eot_upstream(w, B=512)
    cost = dev(M).requires_grad_(True)
    T = bp.EntropicOT.apply(cost, dev(a), dev(b), w.eta)
    (T * dev(G)).sum().backward()
    torch.cuda.synchronize()
    T_ref, _, _ = oracle.eot_project(M.astype(np.float64), a.astype(np.float64), b.astype(np.float64), w.eta)
    assert np.abs(f64(T.detach()) - T_ref).max() <= FWD_TOL
    check_backward(cost.grad, oracle.eot_bwd(T_ref, G.astype(np.float64), a.astype(np.float64),
                                             b.astype(np.float64), w.eta), G.astype(np.float64), T_ref, w.eta)


# -------------------------------------------------------------- full size ---

def test_full_size_workload_sampled():
    """The benchmark workload at its full size and launch configuration: every
    problem converges and meets the residual gate (checked on the GPU in float64);
    a seeded sample of 4096 problems is compared with the oracle one by one."""
    w = W.EOT_WORKLOADS["eot"]
    M, a, b = W.make_eot(w)
    G = W.make_eot_upstream(w)
    print("eot full size B=%d" % w.B, flush=True)
    Md, ad, bd, Gd = dev(M), dev(a), dev(b), dev(G)
    T, dual, iters = bp.eot_plan(Md, ad, bd, w.eta, w.tol, w.max_iter, with_iters=True)
    D = bp.eot_plan_bwd(T, Gd, ad, w.eta)
    torch.cuda.synchronize()
    assert int((iters < 0).sum()) == 0
    Td = T.double()
    res = torch.maximum((Td.sum(2) - ad.double()).abs().amax(1), (Td.sum(1) - bd.double()).abs().amax(1))
    assert res.max().item() <= RES_TOL
    idx = np.sort(np.random.default_rng(70).choice(w.B, 4096, replace=False))
    it = torch.from_numpy(idx).to(DEV)
    T_ref, _, st = oracle.eot_project(M[idx].astype(np.float64), a[idx].astype(np.float64),
                                      b[idx].astype(np.float64), w.eta)
    assert (st >= 0).all()
    assert np.abs(f64(T[it]) - T_ref).max() <= FWD_TOL
    check_backward(D[it], oracle.eot_bwd(T_ref, G[idx].astype(np.float64), a[idx].astype(np.float64),
                                         b[idx].astype(np.float64), w.eta), G[idx].astype(np.float64), T_ref, w.eta)


def test_problems_beyond_32bit_offsets():
    """2^26 + 29 problems of 4 x 6: the cost, plan and gradient arrays are 6.4 GB
    each, so byte offsets pass 2^32 (the benchmark workload stays at 0.4 GB).
    Costs and per-problem marginals (dyadic, summing to exactly one) are drawn on
    the device; the residual of every plan is checked there in float64, and a sample
    that includes the last problems against the oracle."""
    B, n, m, eta = (1 << 26) + 29, 4, 6, 0.5
    print("eot 64-bit offsets B=%d" % B, flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(93)
    def dyadic(k):
        # weights ~ U(0.5, 1.5) turned into multiples of 2^-20 summing to exactly one
        wts = torch.rand((B, k), generator=g, device=DEV) + 0.5
        q = torch.floor(wts / wts.sum(1, keepdim=True) * float(1 << 20))
        q[torch.arange(B, device=DEV), q.argmax(1)] += float(1 << 20) - q.sum(1)
        return q / float(1 << 20)

    M = torch.randn((B, n, m), generator=g, device=DEV)
    a, b = dyadic(n), dyadic(m)
    assert (a.sum(1) == 1).all().item() and (b.sum(1) == 1).all().item()
    G = torch.randn((B, n, m), generator=g, device=DEV)
    T, dual = bp.eot_plan(M, a, b, eta)
    D = bp.eot_plan_bwd(T, G, a, eta)
    torch.cuda.synchronize()
    res, step = 0.0, 1 << 23
    for s in range(0, B, step):
        Td = T[s:s + step].double()
        r = torch.maximum((Td.sum(2) - a[s:s + step].double()).abs().amax(1),
                          (Td.sum(1) - b[s:s + step].double()).abs().amax(1))
        res = max(res, r.max().item())
        assert torch.isfinite(D[s:s + step]).all().item()
    del Td
    assert res <= RES_TOL, res
    rng = np.random.default_rng(94)
    idx = np.unique(np.concatenate([np.arange(B - 64, B), rng.choice(B, 960, replace=False)]))
    it = torch.from_numpy(idx).to(DEV)
    Ms, As, Bs, Gs = f64(M[it]), f64(a[it]), f64(b[it]), f64(G[it])
    T_ref, _, st = oracle.eot_project(Ms, As, Bs, eta)
    assert (st >= 0).all()
    assert np.abs(f64(T[it]) - T_ref).max() <= FWD_TOL
    check_backward(D[it], oracle.eot_bwd(T_ref, Gs, As, Bs, eta), Gs, T_ref, eta)
    del M, G, T, D, dual
    torch.cuda.empty_cache()


@pytest.mark.parametrize("eta", [1.0 / 16, 1.0 / 32])
def test_forward_sharp_plans_verified(eta):
    """Costs N(0, 1) at eta = 1/16 and 1/32: cost spans of 100 to 200 in units of
    eta, so the plan's starting row softmaxes lose entries to fp32 underflow while
    the iteration forms them multiplicatively; a converged plan with entries below
    2^-100 is checked against its dual before it is accepted.  Every problem either
    converges -- then it meets the forward gates against the oracle, where the
    oracle certifies it (all but a few percent at eta = 1/32), and equals the plan
    rebuilt from its dual, eq (4)'s optimality conditions -- or reports -1, exactly
    where its float64 column residual exceeds tol/2.
    The step rule crawls on the sharpest plans (no step size lowers the gradient
    norm, and fallback sweeps move the dual slowly): the cap is 1000 updates, and
    at eta = 1/32 a few percent of the problems still report -1 -- the method's
    limit on such plans, which the test records rather than gates."""
    w = workload(4, 6, eta=eta, seed=71)
    B = 2048
    M, a, b = W.make_eot(w, B=B)
    print("eot sharp eta=%g" % eta, flush=True)
    T, dual, iters = bp.eot_plan(dev(M), dev(a), dev(b), eta, max_iter=1000, with_iters=True)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    conv = it >= 0
    assert conv.mean() >= 0.9, conv.mean()
    M64, a64, b64 = M.astype(np.float64), a.astype(np.float64), b.astype(np.float64)
    Tg, dg = f64(T), f64(dual)
    assert np.isfinite(Tg).all()
    assert residual(Tg, a64, b64)[conv].max() <= RES_TOL
    assert np.abs(rebuilt(M64, a64, dg, eta) - Tg).max(axis=(1, 2))[conv].max() <= FWD_TOL
    assert (np.abs(Tg.sum(1) - b64).max(1)[~conv] > 0.5e-6).all()
    T_ref, _, st = oracle.eot_project(M64, a64, b64, eta)
    cert = st >= 0
    assert (~cert).sum() <= B // 20   # the float64 oracle's own Newton stalls on a few percent at eta = 1/32
    err = np.abs(Tg - T_ref).max(axis=(1, 2))
    assert err[conv & cert].max() <= FWD_TOL, err[conv & cert].max()
    print("  unconverged %d, uncertified %d, max updates %d, err %.2e" % ((~conv).sum(), (~cert).sum(),
                                                                         it.max(), err[conv & cert].max()))


@pytest.mark.parametrize("n", [3, 4, 8])
def test_backward_at_permutation_like_plans(n):
    """eq (13) at plans that are a scaled permutation (one entry per row and column,
    uniform marginals): Delta is zero there, and the exact dcost is zero since such
    a plan does not move under small changes of the cost.  The kernel's solve
    fails, falls back as documented (w = 0), and D is exactly zero, not NaN."""
    rng = np.random.default_rng([n, 72])
    B = 128
    a = np.full(n, 1.0 / n, dtype=np.float32)
    T = np.zeros((B, n, n), dtype=np.float32)
    for k in range(B):
        T[k, np.arange(n), rng.permutation(n)] = 1.0 / n
    G = rng.standard_normal((B, n, n)).astype(np.float32)
    D = bp.eot_plan_bwd(dev(T), dev(G), dev(a), 0.5)
    torch.cuda.synchronize()
    Dg = f64(D)
    assert np.isfinite(Dg).all()
    assert (Dg == 0.0).all(), np.abs(Dg).max()
