"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded inputs.  Needs an MI355X; run with -m gpu.

Gates (fp32 storage):
  forward   max |T - T_ref| <= 1e-5 over every entry, and the same distance between
            T and the T rebuilt in float64 from (logits, dual) -- rows of the
            projection are Softmax(H_i. + beta), so this checks the dual too;
  residual  max(|rowsum - 1|, |colsum - 1|) of the GPU's T, summed in float64, <= 1e-5;
  backward  per matrix max|dH - dH_ref| / max|dH_ref| <= 1e-4.
bf16 storage adds half a bf16 ulp of the reference value to the T and dH gates
(an fp32-exact answer must still be rounded once to be stored), and takes the
residual on T rebuilt in float64 from the logits and the fp32 dual.
On inputs whose projections come near permutations (beyond the five benchmark
workloads) the backward is checked by backward_check instead.
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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def as_storage(a, w):
    """numpy storage array -> device tensor of the ABI's storage dtype."""
    t = dev(a)
    return t.view(torch.bfloat16) if w.io == "bf16" else t


def host_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def half_ulp_bf16(x):
    """Half a bf16 ulp of |x| (bf16 has 8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def residual(T):
    return np.maximum(np.abs(T.sum(axis=-1) - 1).max(axis=-1), np.abs(T.sum(axis=-2) - 1).max(axis=-1))


def rebuilt_T(H, dual):
    """Row softmax of H + beta in float64 (the dual's own projection)."""
    U = H + dual[:, None, :]
    U = U - U.max(axis=2, keepdims=True)
    E = np.exp(U)
    return E / E.sum(axis=2, keepdims=True)


def run_fwd(w, Hs, stats=False):
    """The forward; with stats, birkhoff_fwd_ex and its counts: iters is then the
    pair (updates, fallback sweeps)."""
    B, n = Hs.shape[0], w.n
    H = as_storage(Hs, w)
    T = torch.empty_like(H)
    dual = torch.empty((B, n), dtype=torch.float32, device=DEV)
    iters = None
    if w.io == "bf16":
        bp.birkhoff_fwd_bf16(H, T, dual, w.tol, w.max_iter)
    elif stats:
        it = torch.empty(B, dtype=torch.int32, device=DEV)
        fb = torch.empty(B, dtype=torch.int32, device=DEV)
        bp.birkhoff_fwd_ex(H, T, dual, it, w.tol, w.max_iter, fallbacks=fb)
        iters = (it, fb)
    else:
        bp.birkhoff_fwd(H, T, dual, w.tol, w.max_iter)
    return H, T, dual, iters


def run_bwd(w, H, dual, Gs):
    G = as_storage(Gs, w)
    dH = torch.empty_like(G)
    if w.io == "bf16":
        bp.birkhoff_bwd_bf16(H, dual, G, dH)
    else:
        bp.birkhoff_bwd(H, dual, G, dH)
    return dH


def check_forward(w, H64, T_gpu, dual_gpu, T_ref):
    err = np.abs(T_gpu - T_ref)
    if w.io == "bf16":
        assert (err <= FWD_TOL + half_ulp_bf16(T_ref)).all(), err.max()
        # T rebuilt in float64 from the stored fp32 dual: the dual's own rounding,
        # |beta_j| 2^-24 per entry, moves a column sum by up to about twice its
        # largest (the Hessian's rows have absolute sums of at most 2); four times
        # that is allowed on top of the gate (1e-6 at the benchmark's |beta| ~ 4,
        # 1e-5 at the |beta| ~ 40 of N(0, 10^2) logits)
        r = residual(rebuilt_T(H64, dual_gpu))
        slack = 4.0 * np.abs(dual_gpu).max(axis=1) * U32
        assert (r <= RES_TOL + slack).all(), (r.max(), (r / (RES_TOL + slack)).max())
        res = r.max()
    else:
        assert err.max() <= FWD_TOL, err.max()
        res = residual(T_gpu).max()
        # the dual is the projection's: T rebuilt from it is the returned T
        dd = np.abs(T_gpu - rebuilt_T(H64, dual_gpu)).max()
        assert dd <= FWD_TOL, dd
    assert res <= RES_TOL, res
    return err.max(), res


def check_backward(w, dH_gpu, dH_ref):
    scale = np.abs(dH_ref).max(axis=(1, 2))
    diff = np.abs(dH_gpu - dH_ref)
    if w.io == "bf16":
        ok = diff <= BWD_TOL * scale[:, None, None] + half_ulp_bf16(dH_ref)
        assert ok.all(), diff.max()
        return float((diff.max(axis=(1, 2)) / np.where(scale > 0, scale, 1.0)).max())
    rel = diff.max(axis=(1, 2)) / np.where(scale > 1e-30, scale, 1.0)
    assert rel.max() <= BWD_TOL, rel.max()
    return float(rel.max())


# ----------------------------------------------------- whole-batch parity

@pytest.mark.parametrize("key,B", [("pr1", None), ("train", 8192 + 37), ("n8", 4096 + 19),
                                   ("hard", 8192 + 37), ("bw", 8192 + 37)])
def test_parity_whole_batch(key, B):
    w = W.WORKLOADS[key]
    print("case", key, B, flush=True)
    Hs = W.make_logits(w, B=B)
    H64 = W.decode_f64(Hs)
    H, T, dual, _ = run_fwd(w, Hs)
    T_ref, beta_ref, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    T_gpu = host_f64(T)
    dual_gpu = dual.cpu().numpy().astype(np.float64)
    err, res = check_forward(w, H64, T_gpu, dual_gpu, T_ref)
    assert (dual_gpu[:, -1] == 0).all()
    if key in ("pr1", "train"):   # well-conditioned duals are determined to fp32 accuracy
        assert np.abs(dual_gpu - beta_ref).max() <= 1e-4
    if w.upstream is not None:
        Gs = W.make_upstream(w, B=B)
        dH = run_bwd(w, H, dual, Gs)
        dH_ref = oracle.bwd(T_ref, W.decode_f64(Gs))
        rel = check_backward(w, host_f64(dH), dH_ref)
        print("  fwd err %.2e res %.2e bwd rel %.2e" % (err, res, rel))


# ---------------------------------------------- full sizes, sampled outputs

def sample_indices(B, k=2048, seed=0):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(64, B)), np.arange(max(0, B - 64), B), rng.integers(0, B, k)])
    return np.unique(idx)


@pytest.mark.parametrize("key", ["train", "hard", "n8", "bw"])
def test_parity_full_size_sampled(key):
    """Full batch in the benchmark's launch configuration; the oracle checks a
    sample of matrices one by one and the residual is checked on every output."""
    w = W.WORKLOADS[key]
    print("case full", key, w.B, flush=True)
    Hs = W.make_logits(w)
    H, T, dual, stats = run_fwd(w, Hs, stats=(key == "hard"))
    Gs = W.make_upstream(w) if w.upstream is not None else None
    dH = run_bwd(w, H, dual, Gs) if Gs is not None else None
    torch.cuda.synchronize()
    # residual of every output, in float64 on the device (a property at any size)
    if w.io == "bf16":
        Hd = H.double()
        U = Hd + dual.double()[:, None, :]
        Tr = torch.softmax(U, dim=2)
        res = torch.maximum((Tr.sum(2) - 1).abs().amax(1), (Tr.sum(1) - 1).abs().amax(1)).max().item()
        del Hd, U, Tr
    else:
        Td = T.double()
        res = torch.maximum((Td.sum(2) - 1).abs().amax(1), (Td.sum(1) - 1).abs().amax(1)).max().item()
        del Td
    assert res <= RES_TOL, res
    assert torch.isfinite(T.float()).all().item()
    idx = sample_indices(w.B)
    if stats is not None:
        # matrices that take the fallback sweep (blog post, section 2.2) join the
        # sample (the start's extra sweeps leave the hard inputs few or none; the
        # underflow and large-span tests show the sweep at work)
        its, fbs = stats[0].cpu().numpy(), stats[1].cpu().numpy()
        assert (its >= 0).all() and ((fbs >= 0) & (fbs <= its)).all()
        took = np.flatnonzero(fbs > 0)
        print("  %d matrices took %d fallback sweeps, max updates %d" % (took.size, fbs.sum(), its.max()))
        idx = np.unique(np.concatenate([idx, took[:4096]]))
    it = torch.from_numpy(idx).to(DEV)
    H64 = W.decode_f64(Hs[idx])
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    T_s = host_f64(T[it])
    d_s = dual[it].cpu().numpy().astype(np.float64)
    check_forward(w, H64, T_s, d_s, T_ref)
    if dH is not None:
        dH_ref = oracle.bwd(T_ref, W.decode_f64(Gs[idx]))
        check_backward(w, host_f64(dH[it]), dH_ref)


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("B", [1, 2, 63, 64, 65, 255, 256, 257, 1000])
@pytest.mark.parametrize("n", [4, 8])
def test_ragged_batches_and_canaries(B, n):
    """Outputs land exactly in their slots: padding before and after each output
    buffer keeps its sentinel; results match the oracle."""
    print("case ragged", B, n, flush=True)
    w = W.WORKLOADS["pr1" if n == 4 else "n8"]
    Hs = W.make_logits(w, B=B, seed=1000 + B)
    Gs = W.make_upstream(w, B=B, seed=2000 + B)
    pad = 3
    sentinel = 12345.0
    H = dev(Hs)
    G = dev(Gs)
    Tbuf = torch.full((B + 2 * pad, n, n), sentinel, device=DEV)
    Dbuf = torch.full((B + 2 * pad, n), sentinel, device=DEV)
    Hbuf = torch.full((B + 2 * pad, n, n), sentinel, device=DEV)
    Sbuf = torch.full((B + 2 * pad, n, n), sentinel, device=DEV)
    Ibuf = torch.full((B + 2 * pad,), -7, dtype=torch.int32, device=DEV)
    T, dual, dH, S, it = Tbuf[pad:pad + B], Dbuf[pad:pad + B], Hbuf[pad:pad + B], Sbuf[pad:pad + B], Ibuf[pad:pad + B]
    bp.birkhoff_fwd_ex(H, T, dual, it, w.tol, w.max_iter)
    bp.birkhoff_bwd(H, dual, G, dH)
    bp.sinkhorn_fwd(H, S, 20)
    torch.cuda.synchronize()
    for buf in (Tbuf, Dbuf, Hbuf, Sbuf):
        assert (buf[:pad] == sentinel).all() and (buf[pad + B:] == sentinel).all()
    assert (Ibuf[:pad] == -7).all() and (Ibuf[pad + B:] == -7).all()
    T_ref, _, _ = oracle.project(Hs.astype(np.float64))
    check_forward(w, Hs.astype(np.float64), host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)
    check_backward(w, host_f64(dH), oracle.bwd(T_ref, Gs.astype(np.float64)))
    assert (it.cpu().numpy() >= 0).all()
    np.testing.assert_allclose(host_f64(S), oracle.sinkhorn_k(Hs.astype(np.float64), 20), rtol=0, atol=1e-5)


def test_bf16_ragged_canaries():
    w = W.WORKLOADS["bw"]
    B, pad = 77, 8   # pad of 8 bf16 matrices keeps 16-byte alignment
    Hs = W.make_logits(w, B=B, seed=31)
    Gs = W.make_upstream(w, B=B, seed=32)
    H = as_storage(Hs, w)
    G = as_storage(Gs, w)
    Tbuf = torch.full((B + 2 * pad, 4, 4), 3.0, device=DEV, dtype=torch.bfloat16)
    Hbuf = torch.full((B + 2 * pad, 4, 4), 3.0, device=DEV, dtype=torch.bfloat16)
    dual = torch.empty((B, 4), device=DEV)
    T, dH = Tbuf[pad:pad + B], Hbuf[pad:pad + B]
    bp.birkhoff_fwd_bf16(H, T, dual, w.tol, w.max_iter)
    bp.birkhoff_bwd_bf16(H, dual, G, dH)
    torch.cuda.synchronize()
    for buf in (Tbuf, Hbuf):
        assert (buf[:pad] == 3.0).all() and (buf[pad + B:] == 3.0).all()
    H64 = W.decode_f64(Hs)
    T_ref, _, _ = oracle.project(H64)
    check_forward(w, H64, host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)
    check_backward(w, host_f64(dH), oracle.bwd(T_ref, W.decode_f64(Gs)))


@pytest.mark.parametrize("B", [1, 31, 32, 33, 300, 2007])
def test_bf16_n8_parity_and_canaries(B):
    """bf16 storage for 8x8 matrices (lane pairs, four 16-byte chunks per lane):
    forward, backward and the one-launch forward + backward against the oracle
    at the bf16 gates, with sentinels around every output."""
    print("case bf16 n8 B=%d" % B, flush=True)
    n, pad, sent = 8, 2, 3.0
    w = W.Workload(key="bf16n8", title="8x8 bf16, N(0,1)", B=B, n=n, io="bf16", logits=("normal", 1.0),
                   upstream=("normal", 1.0), passes="fwd+bwd", seed=41)
    Hs = W.make_logits(w, B=B)
    Gs = W.make_upstream(w, B=B)
    H = as_storage(Hs, w)
    G = as_storage(Gs, w)

    def bufs():
        Tb = torch.full((B + 2 * pad, n, n), sent, device=DEV, dtype=torch.bfloat16)
        Hb = torch.full((B + 2 * pad, n, n), sent, device=DEV, dtype=torch.bfloat16)
        Db = torch.full((B + 2 * pad, n), sent, device=DEV)
        return Tb, Hb, Db

    T1b, H1b, D1b = bufs()
    T1, dH1, d1 = T1b[pad:pad + B], H1b[pad:pad + B], D1b[pad:pad + B]
    bp.birkhoff_fwd_bf16(H, T1, d1, w.tol, w.max_iter)
    bp.birkhoff_bwd_bf16(H, d1, G, dH1)
    T2b, H2b, D2b = bufs()
    T2, dH2, d2 = T2b[pad:pad + B], H2b[pad:pad + B], D2b[pad:pad + B]
    bp.birkhoff_fwd_bwd_bf16(H, G, T2, d2, dH2, w.tol, w.max_iter)
    torch.cuda.synchronize()
    for buf in (T1b, H1b, D1b, T2b, H2b, D2b):
        assert (buf[:pad] == sent).all() and (buf[pad + B:] == sent).all()
    # the one-launch form runs the same forward: T and the dual are bit-identical
    assert torch.equal(T1, T2) and torch.equal(d1, d2)
    H64 = W.decode_f64(Hs)
    T_ref, _, st = oracle.project(H64)
    assert (st >= 0).all()
    dH_ref = oracle.bwd(T_ref, W.decode_f64(Gs))
    for T, d, dH in ((T1, d1, dH1), (T2, d2, dH2)):
        check_forward(w, H64, host_f64(T), d.cpu().numpy().astype(np.float64), T_ref)
        assert (d[:, -1] == 0).all().item()
        check_backward(w, host_f64(dH), dH_ref)


def test_empty_batch_is_a_noop():
    H = torch.empty((0, 4, 4), device=DEV)
    T, dual = bp.project(H)
    assert T.shape == (0, 4, 4) and dual.shape == (0, 4)
    assert bp.project_bwd(H, dual, torch.empty((0, 4, 4), device=DEV)).shape == (0, 4, 4)
    assert bp.sinkhorn(H).shape == (0, 4, 4)


@pytest.mark.parametrize("n", [4, 8])
def test_special_inputs(n):
    """Exactly known projections: doubly stochastic inputs with row/column shifts
    map to themselves, rank-one inputs map to J/n, constant inputs to J/n."""
    rng = np.random.default_rng(5)
    B = 300
    P = np.empty((B, n, n))
    for b in range(B):
        wts = rng.dirichlet(np.ones(5))
        M = np.zeros((n, n))
        for k in range(5):
            M[np.arange(n), rng.permutation(n)] += wts[k]
        P[b] = 0.9 * M + 0.1 / n
    a, c = rng.standard_normal((B, n, 1)), rng.standard_normal((B, 1, n))
    H = (np.log(P) + a + c).astype(np.float32)
    T, dual = bp.project(dev(H))
    np.testing.assert_allclose(host_f64(T), P, rtol=0, atol=2e-5)
    R = (a + c + np.zeros((1, n, n))).astype(np.float32)
    T1, _ = bp.project(dev(R))
    np.testing.assert_allclose(host_f64(T1), 1.0 / n, rtol=0, atol=1e-6)
    T0, d0 = bp.project(torch.zeros((5, n, n), device=DEV))
    assert (host_f64(T0) == 1.0 / n).all() and (d0.cpu().numpy() == 0).all()


def test_nonfinite_inputs_stay_in_their_matrix():
    w = W.WORKLOADS["pr1"]
    Hs = W.make_logits(w, B=300)
    bad = Hs.copy()
    bad[5, 1, 2] = np.nan
    bad[9, 0, 0] = np.inf
    bad[200, 3, 3] = -np.inf
    T0, d0 = bp.project(dev(Hs))
    T1, d1 = bp.project(dev(bad))
    torch.cuda.synchronize()
    t0, t1 = T0.cpu().numpy(), T1.cpu().numpy()
    keep = np.setdiff1d(np.arange(300), [5, 9, 200])
    assert np.array_equal(t0[keep], t1[keep])
    assert np.isnan(t1[5]).any() and np.isnan(t1[9]).any()
    iters = torch.empty(300, dtype=torch.int32, device=DEV)
    T2 = torch.empty_like(T1)
    d2 = torch.empty_like(d1)
    bp.birkhoff_fwd_ex(dev(bad), T2, d2, iters)
    assert iters[5].item() == -1 and iters[9].item() == -1


def test_max_iter_one_and_stats():
    w = W.WORKLOADS["hard"]
    Hs = W.make_logits(w, B=4096)
    H = dev(Hs)
    T = torch.empty_like(H)
    dual = torch.empty((4096, 4), device=DEV)
    it = torch.empty(4096, dtype=torch.int32, device=DEV)
    bp.birkhoff_fwd_ex(H, T, dual, it, 1e-6, 1)
    assert torch.isfinite(T).all().item()
    assert ((it == -1) | (it <= 1)).all().item()
    bp.birkhoff_fwd_ex(H, T, dual, it, w.tol, w.max_iter)
    itn = it.cpu().numpy()
    assert (itn >= 0).all(), (itn < 0).sum()        # every hard matrix converges within 100 updates
    T2 = torch.empty_like(T)
    bp.birkhoff_fwd(H, T2, torch.empty_like(dual), w.tol, w.max_iter)
    assert torch.equal(T, T2)                        # the stats variant computes the same thing
    print("iterations: mean %.2f max %d" % (itn.mean(), itn.max()))


def test_repeatable_and_stream_ordered():
    w = W.WORKLOADS["train"]
    Hs = W.make_logits(w, B=50_000)
    Gs = W.make_upstream(w, B=50_000)
    H, G = dev(Hs), dev(Gs)
    T1, d1 = bp.project(H)
    dH1 = bp.project_bwd(H, d1, G)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        T2, d2 = bp.project(H)
        dH2 = bp.project_bwd(H, d2, G)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(T1, T2) and torch.equal(d1, d2) and torch.equal(dH1, dH2)


@pytest.mark.parametrize("key", ["pr1", "n8", "bw"])
def test_autograd_function_matches_oracle(key):
    """torch.autograd through BirkhoffProjection: fp32 differentiates from the saved
    T (birkhoff_bwd_from_T), bf16 storage from the saved logits and dual."""
    w = W.WORKLOADS[key]
    Hs = W.make_logits(w, B=512 + 7)
    Gs = W.make_upstream(w, B=512 + 7)
    H = as_storage(Hs, w).requires_grad_(True)
    T = bp.BirkhoffProjection.apply(H)
    (T * as_storage(Gs, w)).sum().backward()
    H64 = W.decode_f64(Hs)
    T_ref, _, _ = oracle.project(H64)
    err = np.abs(host_f64(T.detach()) - T_ref)
    assert (err <= FWD_TOL + (half_ulp_bf16(T_ref) if w.io == "bf16" else 0.0)).all(), err.max()
    check_backward(w, host_f64(H.grad), oracle.bwd(T_ref, W.decode_f64(Gs)))


@pytest.mark.parametrize("K", [1, 5, 20])
@pytest.mark.parametrize("key", ["pr1", "hard", "n8"])
def test_sinkhorn_baseline_matches_oracle(key, K):
    w = W.WORKLOADS[key]
    Hs = W.make_logits(w, B=4096 + 13)
    T = bp.sinkhorn(dev(Hs), K)
    ref = oracle.sinkhorn_k(Hs.astype(np.float64), K)
    np.testing.assert_allclose(host_f64(T), ref, rtol=0, atol=1e-5)


def test_newton_versus_sinkhorn20_on_hard_inputs():
    """The pages' qualitative claim (section 5): at large magnitudes 20 Sinkhorn sweeps
    leave large marginal errors, while Newton's stay small (L1 of row and column sums)."""
    w = W.WORKLOADS["hard"]
    Hs = W.make_logits(w, B=65536)
    H = dev(Hs)
    T, _ = bp.project(H, w.tol, w.max_iter)
    S = bp.sinkhorn(H, 20)
    l1 = lambda X: ((X.double().sum(2) - 1).abs().sum(1) + (X.double().sum(1) - 1).abs().sum(1))
    e_newton, e_sk = l1(T), l1(S)
    print("L1 marginal error: newton max %.2e median %.2e | SK-20 max %.2e median %.2e" % (
        e_newton.max().item(), e_newton.median().item(), e_sk.max().item(), e_sk.median().item()))
    assert e_newton.max().item() < 1e-4
    assert e_sk.max().item() > 100 * e_newton.max().item()


# ------------------------------------------- forward + backward in one launch

def run_fused(w, Hs, Gs):
    B, n = Hs.shape[0], w.n
    H = as_storage(Hs, w)
    G = as_storage(Gs, w)
    T = torch.empty_like(H)
    dH = torch.empty_like(G)
    dual = torch.empty((B, n), dtype=torch.float32, device=DEV)
    if w.io == "bf16":
        bp.birkhoff_fwd_bwd_bf16(H, G, T, dual, dH, w.tol, w.max_iter)
    else:
        bp.birkhoff_fwd_bwd(H, G, T, dual, dH, w.tol, w.max_iter)
    return H, G, T, dual, dH


@pytest.mark.parametrize("key,B", [("pr1", None), ("train", 8192 + 37), ("n8", 4096 + 19), ("bw", 8192 + 37)])
def test_fused_parity_and_agreement_with_separate_calls(key, B):
    """One-launch forward + backward against the oracle; its T and dual are the
    separate forward's bit for bit, its dH agrees with the separate backward."""
    w = W.WORKLOADS[key]
    print("case fused", key, B, flush=True)
    Hs = W.make_logits(w, B=B)
    Gs = W.make_upstream(w, B=B)
    H64 = W.decode_f64(Hs)
    H, G, T, dual, dH = run_fused(w, Hs, Gs)
    _, T2, dual2, _ = run_fwd(w, Hs)
    dH2 = run_bwd(w, H, dual2, Gs)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    check_forward(w, H64, host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)
    dH_ref = oracle.bwd(T_ref, W.decode_f64(Gs))
    rel = check_backward(w, host_f64(dH), dH_ref)
    rel2 = check_backward(w, host_f64(dH2), dH_ref)
    print("  fused bwd rel %.2e, separate bwd rel %.2e" % (rel, rel2))


@pytest.mark.parametrize("key", ["train", "bw"])
def test_fused_full_size_sampled(key):
    w = W.WORKLOADS[key]
    print("case fused full", key, w.B, flush=True)
    Hs = W.make_logits(w)
    Gs = W.make_upstream(w)
    H, G, T, dual, dH = run_fused(w, Hs, Gs)
    torch.cuda.synchronize()
    assert torch.isfinite(T.float()).all().item() and torch.isfinite(dH.float()).all().item()
    idx = sample_indices(w.B)
    it = torch.from_numpy(idx).to(DEV)
    H64 = W.decode_f64(Hs[idx])
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    check_forward(w, H64, host_f64(T[it]), dual[it].cpu().numpy().astype(np.float64), T_ref)
    check_backward(w, host_f64(dH[it]), oracle.bwd(T_ref, W.decode_f64(Gs[idx])))


@pytest.mark.parametrize("B", [1, 63, 64, 65, 257])
@pytest.mark.parametrize("n", [4, 8])
def test_fused_ragged_batches_and_canaries(B, n):
    print("case fused ragged", B, n, flush=True)
    w = W.WORKLOADS["pr1" if n == 4 else "n8"]
    Hs = W.make_logits(w, B=B, seed=3000 + B)
    Gs = W.make_upstream(w, B=B, seed=4000 + B)
    pad, sentinel = 3, -777.0
    bufs = [torch.full((B + 2 * pad, n, n), sentinel, device=DEV) for _ in range(2)]
    Dbuf = torch.full((B + 2 * pad, n), sentinel, device=DEV)
    T, dH, dual = bufs[0][pad:pad + B], bufs[1][pad:pad + B], Dbuf[pad:pad + B]
    bp.birkhoff_fwd_bwd(dev(Hs), dev(Gs), T, dual, dH, w.tol, w.max_iter)
    torch.cuda.synchronize()
    for buf in bufs + [Dbuf]:
        assert (buf[:pad] == sentinel).all() and (buf[pad + B:] == sentinel).all()
    H64 = Hs.astype(np.float64)
    T_ref, _, _ = oracle.project(H64)
    check_forward(w, H64, host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)
    check_backward(w, host_f64(dH), oracle.bwd(T_ref, Gs.astype(np.float64)))


def test_fused_empty_batch_is_a_noop():
    H = torch.empty((0, 4, 4), device=DEV)
    T, dual, dH = bp.project_fwd_bwd(H, torch.empty((0, 4, 4), device=DEV))
    assert T.shape == (0, 4, 4) and dual.shape == (0, 4) and dH.shape == (0, 4, 4)


# ------------------------------------------------ backward from (T*, G) only

@pytest.mark.parametrize("key,B", [("pr1", None), ("train", 8192 + 37), ("n8", 4096 + 19)])
def test_bwd_from_T_matches_oracle_and_dual_backward(key, B):
    """dH from the projection T and dL/dT alone ([P] section 4.2) against the
    oracle's eq (13) at the reference T, and against the dual-based backward."""
    w = W.WORKLOADS[key]
    print("case bwd_from_T", key, B, flush=True)
    Hs = W.make_logits(w, B=B)
    Gs = W.make_upstream(w, B=B)
    H, T, dual, _ = run_fwd(w, Hs)
    G = dev(Gs)
    dH = torch.empty_like(G)
    bp.birkhoff_bwd_from_T(T, G, dH)
    dH2 = run_bwd(w, H, dual, Gs)
    torch.cuda.synchronize()
    T_ref, _, _ = oracle.project(W.decode_f64(Hs), sk_cap=w.sk_cap)
    dH_ref = oracle.bwd(T_ref, W.decode_f64(Gs))
    rel = check_backward(w, host_f64(dH), dH_ref)
    d = np.abs(host_f64(dH) - host_f64(dH2)).max(axis=(1, 2)) / np.abs(dH_ref).max(axis=(1, 2))
    assert d.max() <= 2 * BWD_TOL
    print("  from-T bwd rel %.2e, vs dual-based %.2e" % (rel, d.max()))


@pytest.mark.parametrize("B", [1, 65, 257])
def test_bwd_from_T_ragged_canaries(B):
    w = W.WORKLOADS["pr1"]
    Hs = W.make_logits(w, B=B, seed=5000 + B)
    Gs = W.make_upstream(w, B=B, seed=6000 + B)
    T_ref, _, _ = oracle.project(Hs.astype(np.float64))
    pad, sentinel = 3, 99.0
    buf = torch.full((B + 2 * pad, 4, 4), sentinel, device=DEV)
    dH = buf[pad:pad + B]
    bp.birkhoff_bwd_from_T(dev(T_ref.astype(np.float32)), dev(Gs), dH)
    torch.cuda.synchronize()
    assert (buf[:pad] == sentinel).all() and (buf[pad + B:] == sentinel).all()
    check_backward(w, host_f64(dH), oracle.bwd(T_ref, Gs.astype(np.float64)))


def test_near_singular_hessian_does_not_stall():
    """Two matrices of the hard workload whose Newton Hessian has an eigenvalue
    below fp32 resolution (a column carried by one entry near 1): without the
    sub-resolution shift of the Newton system they needed 86 and more than 200
    updates; now they converge like their neighbours, to the oracle's T."""
    w = W.WORKLOADS["hard"]
    idx = np.array([164138, 1020551])
    Hs = W.make_logits(w)[idx]
    H = dev(Hs)
    T = torch.empty_like(H)
    dual = torch.empty((2, 4), device=DEV)
    it = torch.empty(2, dtype=torch.int32, device=DEV)
    bp.birkhoff_fwd_ex(H, T, dual, it, w.tol, w.max_iter)
    itn = it.cpu().numpy()
    print("iterations", itn)
    assert (itn >= 0).all() and itn.max() <= 30
    T_ref, _, st = oracle.project(Hs.astype(np.float64), sk_cap=w.sk_cap)
    assert (st >= 0).all()
    check_forward(w, Hs.astype(np.float64), host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)


# ------------------------------------- slow lanes gathered across the workgroup

# Slow lanes (still running after the first four updates) per wave of 64, four
# waves to a workgroup: hand-offs that fill one or two waves, waves that keep
# their slow lanes (more than 32), mixtures, an idle workgroup, and a last
# workgroup with a partial wave and three empty ones.
GATHER_WAVES = [32, 32, 32, 32,
                64, 0, 0, 1,
                33, 32, 5, 64,
                0, 0, 0, 0,
                17, 63, 2, 21,
                31, 33, 20, 1]
GATHER_TAIL = (40, 20)   # a last wave of 40 matrices, 20 of them slow


def gather_batch(seed=90):
    """Logits laid out by GATHER_WAVES: "slow" matrices take >= 8 float64 Newton
    updates in the oracle (N(0, 8^2) logits), "fast" ones <= 2 (N(0, 0.5^2) + 2I)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = (rng.standard_normal((12000, 4, 4)) * 8.0).astype(np.float32)
    _, _, it = oracle.newton(pool.astype(np.float64), tol=1e-6, max_iter=100)
    slow = list(pool[it >= 8])
    easy = (rng.standard_normal((4000, 4, 4)) * 0.5 + 2.0 * np.eye(4)).astype(np.float32)
    _, _, it = oracle.newton(easy.astype(np.float64), tol=1e-6, max_iter=100)
    fast = list(easy[(it >= 0) & (it <= 2)])
    waves = [(64, s) for s in GATHER_WAVES] + [GATHER_TAIL]
    out, want_slow = [], []
    for size, s in waves:
        pos = set(rng.choice(size, s, replace=False).tolist())
        for lane in range(size):
            out.append(slow.pop() if lane in pos else fast.pop())
            want_slow.append(lane in pos)
    return np.stack(out), np.array(want_slow)


@pytest.mark.parametrize("max_iter", [100, 5, 4])
def test_gathered_slow_lanes(max_iter):
    """The n = 4 forward hands the slow lanes of a wave to other waves of its
    workgroup: every layout of slow lanes gives the oracle's projection, and the
    same T and dual, bit for bit, as the fused kernel (which runs every matrix to
    the end in its own lane)."""
    Hs, want_slow = gather_batch()
    B = Hs.shape[0]
    print("case gather B=%d max_iter=%d" % (B, max_iter), flush=True)
    H = dev(Hs)
    T = torch.empty_like(H)
    dual = torch.empty((B, 4), device=DEV)
    iters = torch.empty(B, dtype=torch.int32, device=DEV)
    bp.birkhoff_fwd_ex(H, T, dual, iters, 1e-6, max_iter)
    T2, d2, dH = torch.empty_like(H), torch.empty_like(dual), torch.empty_like(H)
    bp.birkhoff_fwd_bwd(H, dev(np.ones_like(Hs)), T2, d2, dH, 1e-6, max_iter)
    T3, d3 = torch.empty_like(H), torch.empty_like(dual)
    bp.birkhoff_fwd(H, T3, d3, 1e-6, max_iter)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, d2)
    assert torch.equal(T, T3) and torch.equal(dual, d3)
    it = iters.cpu().numpy()
    assert ((it == -1) | ((it >= 0) & (it <= max_iter))).all()
    if max_iter == 100:
        # the layout is the intended one: fast matrices are done within the first
        # pass, and slow ones (>= 8 float64 updates from the oracle's start) still
        # need more than 4 updates after the kernel's start, which sweeps a lane
        # further while its residual is large -- all but a few of them
        assert (it >= 0).all()
        assert (it[~want_slow] <= 4).all()
        assert (it[want_slow] > 4).mean() >= 0.9, (it[want_slow] > 4).mean()
        T_ref, _, st = oracle.project(Hs.astype(np.float64))
        assert (st >= 0).all()
        check_forward(W.WORKLOADS["hard"], Hs.astype(np.float64), host_f64(T), host_f64(dual), T_ref)
    else:
        assert (it[~want_slow] >= 0).all()



@pytest.mark.parametrize("max_iter", [100, 5])
def test_gathered_slow_lanes_bf16(max_iter):
    """The same layouts in bf16 storage (the slow / fast split of the fp32 pool
    mostly survives the rounding): the gathering forward's T and dual equal the
    fused kernel's bit for bit and pass the bf16 gates against the oracle."""
    Hf, _ = gather_batch()
    Hs = W.f32_to_bf16_bits(Hf)
    B = Hs.shape[0]
    print("case gather bf16 B=%d max_iter=%d" % (B, max_iter), flush=True)
    w = W.WORKLOADS["bw"]
    H = dev(Hs).view(torch.bfloat16)
    T = torch.empty_like(H)
    dual = torch.empty((B, 4), device=DEV)
    bp.birkhoff_fwd_bf16(H, T, dual, 1e-6, max_iter)
    T2, d2, dH = torch.empty_like(H), torch.empty_like(dual), torch.empty_like(H)
    G = dev(W.f32_to_bf16_bits(np.ones_like(Hf))).view(torch.bfloat16)
    bp.birkhoff_fwd_bwd_bf16(H, G, T2, d2, dH, 1e-6, max_iter)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, d2)
    if max_iter == 100:
        H64 = W.decode_f64(Hs)
        T_ref, _, st = oracle.project(H64)
        assert (st >= 0).all()
        check_forward(w, H64, host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)

U32 = 2.0 ** -24   # fp32 unit roundoff


def delta_lambda_min(T):
    """Smallest eigenvalue of eq (13)'s Delta at T, in float64: the Hessian
    diag(c) - T_{-n}^T T_{-n} with its diagonal formed as sum_i T_ij sum_{l != j} T_il
    (no cancellation, so that it keeps its digits near permutations)."""
    m = T.shape[2] - 1
    Gm = np.einsum("bij,bik->bjk", T, T)
    D = -Gm[:, :m, :m].copy()
    for j in range(m):
        D[:, j, j] = Gm[:, j, :].sum(1) - Gm[:, j, j]
    return np.linalg.eigvalsh(D)[:, 0]


def colres(T):
    return np.abs(T.sum(axis=1) - 1).max(axis=1)


def backward_check(dH_gpu, T_used, G, T_ref, where=""):
    """The backward on inputs whose projections come near permutations, where
    eq (13) is ill-conditioned (the smallest eigenvalue lambda of Delta reaches
    1e-11 on the pages' N(0, 10^2) inputs) and dH can be orders of magnitude
    smaller than its terms G o T, which cancel.
    (a) Against eq (13) evaluated by the oracle at the T the kernel used (T_used:
        the stored T, or for birkhoff_bwd the T rebuilt from the dual), per matrix
          |dH - dH_ref|_max <= 1e-4 |dH_ref|_max + |G o T|_max (8 n u + r) / lambda,
        u = 2^-24 and r = max_j |c_j - 1| of T_used.  To first order the kernel's
        rounding of Delta (a few ulps per entry, 2(n-1) 2u in norm) and of the
        right-hand side mu_c - T^T mu_r (about 4 n u |G o T|) reach dH through
        Delta^-1; the kernel's Delta is the Hessian at T_used, diag(c) - T^T T,
        the oracle's the literal I - T^T T, and they differ by r.  Wherever lambda
        exceeds about 3e-4 this gate is below 1e-2 |G o T| (typically far below).
    (b) Against eq (13) at the reference projection T_ref, the gate widened by the
        measured forward error d = |T_used - T_ref|_max: 2(n-1) d more in Delta's
        norm, and 2 |G|_max d for the factor T of dH itself.
    (c) At any conditioning: T does not change when a constant is added to a row
        or a column of H, so every row and every column of the exact dH sums to
        zero.  The kernel's column sums are the residual of its Delta solve --
        rounding level, or, where Delta is below fp32 resolution and is solved
        with 2^-20 (1 + tr Delta) added, that shift times w, which the shift keeps
        within a few |G| -- and its row sums (1 - rowsum(T)) times O(|G| + |w|);
        both stay within 1e-4 |G|_max.
    The oracle's literal Delta = I - T^T T differs from the Hessian at T by
    diag(c - 1), so it is positive definite only where lambda exceeds the
    column residual r; below that (lambda under 1e-7 at the GPU's T, 1e-13 at
    T_ref) its eq (13) is no reference, and those matrices are checked by (c)
    only.  Returns (number of matrices where (a)'s gate is above 1e-2 |G o T|,
    largest ratio of error to gate in (a))."""
    n = T_used.shape[2]
    gt = np.abs(G * T_used).max(axis=(1, 2))
    lam = np.maximum(delta_lambda_min(T_used), 1e-300)
    ref = oracle.bwd(T_used, G)
    fin = np.isfinite(ref).all(axis=(1, 2)) & (lam > 2 * colres(T_used) + 1e-12)
    err = np.abs(dH_gpu - ref).max(axis=(1, 2))
    gate = 1e-4 * np.abs(ref).max(axis=(1, 2)) + gt * (8 * n * U32 + colres(T_used)) / lam
    ratio = np.where(fin, err / gate, 0.0)
    assert (ratio <= 1.0).all(), "%s (a): error %.3e above gate %.3e (lambda %.3e, |GoT| %.3e)" % (
        where, err[np.argmax(ratio)], gate[np.argmax(ratio)], lam[np.argmax(ratio)], gt[np.argmax(ratio)])
    ref2 = oracle.bwd(T_ref, G)
    fin2 = fin & np.isfinite(ref2).all(axis=(1, 2)) & (delta_lambda_min(T_ref) > 2 * colres(T_ref) + 1e-12)
    d = np.abs(T_used - T_ref).max(axis=(1, 2))
    err2 = np.abs(dH_gpu - ref2).max(axis=(1, 2))
    gate2 = (1e-4 * np.abs(ref2).max(axis=(1, 2)) + gt * (8 * n * U32 + colres(T_used) + 2 * (n - 1) * d) / lam
             + 2 * np.abs(G).max(axis=(1, 2)) * d)
    ratio2 = np.where(fin2, err2 / gate2, 0.0)
    assert (ratio2 <= 1.0).all(), "%s (b): error %.3e above gate %.3e" % (
        where, err2[np.argmax(ratio2)], gate2[np.argmax(ratio2)])
    assert np.isfinite(dH_gpu).all(), where
    gmax = np.abs(G).max(axis=(1, 2))
    rows = np.abs(dH_gpu.sum(axis=2)).max(axis=1) / gmax
    cols = np.abs(dH_gpu.sum(axis=1)).max(axis=1) / gmax
    assert rows.max() <= 1e-4 and cols.max() <= 1e-4, "%s (c): row sums %.2e, column sums %.2e of |G|" % (
        where, rows.max(), cols.max())
    return int((gate > 1e-2 * gt).sum()), float(ratio.max())


@pytest.mark.parametrize("B", [512, 8192])
def test_parity_pages_timing_shape(B):
    """The pages' timing inputs (4x4, N(0, 10^2) logits: farther from uniform than any
    benchmark workload) through the forward (gathering kernel), the backward and the
    one-launch forward + backward, against the oracle.  Many of these projections are
    nearly permutations, where eq (13) is ill-conditioned; the backward is checked
    by backward_check.  Matrices that take the fallback sweep (blog post, section
    2.2) meet the gates like the rest; the start's extra sweeps leave these inputs
    few or none (the underflow and large-span tests show the sweep at work)."""
    w = W.pages_shape_workload(B)
    print("case pages shape", B, flush=True)
    Hs = W.make_logits(w)
    Gs = W.make_upstream(w)
    H64 = Hs.astype(np.float64)
    H, T, dual, (iters, fb) = run_fwd(w, Hs, stats=True)
    dH = run_bwd(w, H, dual, Gs)
    _, _, T2, dual2, dH2 = run_fused(w, Hs, Gs)
    dH3 = torch.empty_like(dH)
    bp.birkhoff_bwd_from_T(T2, dev(Gs), dH3)
    torch.cuda.synchronize()
    it, fbn = iters.cpu().numpy(), fb.cpu().numpy()
    assert (it >= 0).all(), (it < 0).sum()
    assert ((fbn >= 0) & (fbn <= it)).all()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    Tg, dg = host_f64(T), host_f64(dual)
    err, res = check_forward(w, H64, Tg, dg, T_ref)
    G64 = Gs.astype(np.float64)
    loose, r1 = backward_check(host_f64(dH), rebuilt_T(H64, dg), G64, T_ref, "bwd")
    _, r2 = backward_check(host_f64(dH2), Tg, G64, T_ref, "fused")
    _, r3 = backward_check(host_f64(dH3), Tg, G64, T_ref, "from_T")
    fb_err = np.abs(Tg - T_ref)[fbn > 0].max() if (fbn > 0).any() else 0.0
    print("  max updates %d, %d matrices took %d fallback sweeps; fwd err %.2e (fallback matrices %.2e), "
          "residual %.2e; bwd worst error/gate %.2f / %.2f / %.2f, %d of %d with a loose gate" % (
              it.max(), (fbn > 0).sum(), fbn.sum(), err, fb_err, res, r1, r2, r3, loose, B))


@pytest.mark.parametrize("B", [1, 65, 257, 1000, 1320])
def test_gathered_ragged_batches_and_canaries(B):
    """Slow matrices (the gathered path's per-lane stores) in ragged batches: every
    output lands in its slot and the padding around each buffer keeps its sentinel."""
    print("case gather ragged", B, flush=True)
    Hs = gather_batch()[0][:B]
    pad, sentinel = 3, 12345.0
    Tbuf = torch.full((B + 2 * pad, 4, 4), sentinel, device=DEV)
    Dbuf = torch.full((B + 2 * pad, 4), sentinel, device=DEV)
    Ibuf = torch.full((B + 2 * pad,), -7, dtype=torch.int32, device=DEV)
    T, dual, it = Tbuf[pad:pad + B], Dbuf[pad:pad + B], Ibuf[pad:pad + B]
    bp.birkhoff_fwd_ex(dev(Hs), T, dual, it, 1e-6, 100)
    torch.cuda.synchronize()
    for buf in (Tbuf, Dbuf):
        assert (buf[:pad] == sentinel).all() and (buf[pad + B:] == sentinel).all()
    assert (Ibuf[:pad] == -7).all() and (Ibuf[pad + B:] == -7).all()
    assert (it.cpu().numpy() >= 0).all()
    T_ref, _, _ = oracle.project(Hs.astype(np.float64))
    check_forward(W.WORKLOADS["hard"], Hs.astype(np.float64), host_f64(T), host_f64(dual), T_ref)


def test_gathered_nonfinite_inputs_stay_in_their_matrix():
    """Non-finite logits among slow matrices: the bad matrices end with count -1 and
    every other matrix's T and dual are those of the clean batch, bit for bit."""
    Hs, want_slow = gather_batch()
    bad = Hs.copy()
    slow_idx = np.flatnonzero(want_slow)
    hit = [int(slow_idx[3]), int(slow_idx[40]), 7, int(slow_idx[200])]
    bad[hit[0], 1, 2] = np.nan
    bad[hit[1], 0, 0] = np.inf
    bad[hit[2], 2, 1] = np.nan
    bad[hit[3], 3, 3] = np.inf
    B = Hs.shape[0]
    out = []
    for X in (Hs, bad):
        T = torch.empty((B, 4, 4), device=DEV)
        d = torch.empty((B, 4), device=DEV)
        it = torch.empty(B, dtype=torch.int32, device=DEV)
        bp.birkhoff_fwd_ex(dev(X), T, d, it, 1e-6, 100)
        out.append((T.cpu().numpy(), d.cpu().numpy(), it.cpu().numpy()))
    keep = np.setdiff1d(np.arange(B), hit)
    assert np.array_equal(out[0][0][keep], out[1][0][keep])
    assert np.array_equal(out[0][1][keep], out[1][1][keep])
    assert np.array_equal(out[0][2][keep], out[1][2][keep])
    assert (out[1][2][hit] == -1).all()


def test_graph_capture_and_replay():
    """The entry points launch on the stream they are given, allocate nothing and
    record no memset, so a step can be captured into a HIP graph: every replay,
    with the program's own eager work and synchronisations in between, gives the
    eager results bit for bit."""
    w = W.WORKLOADS["pr1"]
    Hs, Gs = W.make_logits(w), W.make_upstream(w)
    H, G = dev(Hs), dev(Gs)
    B = Hs.shape[0]
    T0, d0, dH0 = torch.empty_like(H), torch.empty((B, 4), device=DEV), torch.empty_like(H)
    bp.birkhoff_fwd_bwd(H, G, T0, d0, dH0, w.tol, w.max_iter)
    T1, d1, dH1 = torch.empty_like(H), torch.empty((B, 4), device=DEV), torch.empty_like(H)
    dH2 = torch.empty_like(H)
    Tf, df = torch.empty_like(H), torch.empty((B, 4), device=DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bp.birkhoff_fwd_bwd(H, G, T1, d1, dH1, w.tol, w.max_iter)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bp.birkhoff_fwd_bwd(H, G, T1, d1, dH1, w.tol, w.max_iter)
        bp.birkhoff_fwd(H, Tf, df, w.tol, w.max_iter)
        bp.birkhoff_bwd(H, df, G, dH2)
    T_e, d_e = torch.empty_like(H), torch.empty((B, 4), device=DEV)
    bp.birkhoff_fwd(H, T_e, d_e, w.tol, w.max_iter)
    dH_e = torch.empty_like(H)
    bp.birkhoff_bwd(H, d_e, G, dH_e)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (T1, d1, dH1, Tf, df, dH2):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(T1, T0) and torch.equal(d1, d0) and torch.equal(dH1, dH0), rep
        assert torch.equal(Tf, T_e) and torch.equal(df, d_e) and torch.equal(dH2, dH_e), rep
        bp.project(H)   # eager work between replays
        torch.cuda.synchronize()



def test_parity_n8_large_logits():
    """8x8 logits N(0, s^2) with s per matrix from {1, 3, 5, 8} (the hard workload's
    scales at n = 8): the forward, the backward and the one-launch forward +
    backward against the oracle (backward as backward_check)."""
    w = W.Workload(key="n8_sigma_mix", title="8x8 fp32, H~N(0,s^2), s per matrix from {1,3,5,8}",
                   B=4096 + 19, n=8, io="f32", logits=("sigma_mix", (1.0, 3.0, 5.0, 8.0)),
                   upstream=("normal", 1.0), passes="fwd+bwd", seed=9, max_iter=100, sk_cap=5_000)
    print("case n8 large logits", flush=True)
    Hs, Gs = W.make_logits(w), W.make_upstream(w)
    H64 = Hs.astype(np.float64)
    H, T, dual, (iters, fb) = run_fwd(w, Hs, stats=True)
    dH = run_bwd(w, H, dual, Gs)
    _, _, T2, dual2, dH2 = run_fused(w, Hs, Gs)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    assert (it >= 0).all(), (it < 0).sum()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    Tg, dg = host_f64(T), host_f64(dual)
    err, res = check_forward(w, H64, Tg, dg, T_ref)
    G64 = Gs.astype(np.float64)
    loose, r1 = backward_check(host_f64(dH), rebuilt_T(H64, dg), G64, T_ref, "bwd")
    _, r2 = backward_check(host_f64(dH2), Tg, G64, T_ref, "fused")
    print("  max updates %d, fallback matrices %d, fwd err %.2e, residual %.2e, bwd worst error/gate %.2f / %.2f, "
          "%d with a loose gate" % (it.max(), (fb.cpu().numpy() > 0).sum(), err, res, r1, r2, loose))


def test_batch_beyond_32bit_offsets():
    """2^27 + 37 matrices, so element offsets pass 2^31 and byte offsets 2^32 (the
    largest workload stays below both): the one-launch forward + backward on
    N(0, 1) inputs drawn on the device; every output's residual is checked on the
    device, and a sample that includes the first and the last matrices against
    the oracle."""
    B, n = (1 << 27) + 37, 4
    w = W.WORKLOADS["pr1"]
    print("case 64-bit offsets B=%d" % B, flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    H = torch.randn((B, n, n), generator=g, device=DEV)
    G = torch.randn((B, n, n), generator=g, device=DEV)
    T, dH = torch.empty_like(H), torch.empty_like(H)
    dual = torch.empty((B, n), device=DEV)
    bp.birkhoff_fwd_bwd(H, G, T, dual, dH, w.tol, w.max_iter)
    torch.cuda.synchronize()
    res, step = 0.0, 1 << 24
    for s in range(0, B, step):
        Td = T[s:s + step].double()
        res = max(res, torch.maximum((Td.sum(2) - 1).abs().amax(1), (Td.sum(1) - 1).abs().amax(1)).max().item())
        assert torch.isfinite(dH[s:s + step]).all().item()
        assert (dual[s:s + step, -1] == 0).all().item()
    del Td
    assert res <= RES_TOL, res
    idx = sample_indices(B, k=1024, seed=3)
    it = torch.from_numpy(idx).to(DEV)
    H64 = H[it].cpu().numpy().astype(np.float64)
    T_ref, _, st = oracle.project(H64)
    assert (st >= 0).all()
    check_forward(w, H64, host_f64(T[it]), dual[it].cpu().numpy().astype(np.float64), T_ref)
    check_backward(w, host_f64(dH[it]), oracle.bwd(T_ref, G[it].cpu().numpy().astype(np.float64)))
    del H, G, T, dH, dual
    torch.cuda.empty_cache()


SWEEP_KINDS = ["normal:0.1", "normal:1", "normal:3", "normal:5", "normal:8", "normal:10", "unif:1", "unif:10",
               "nearI", "lowrank", "mix"]


def sweep_logits(kind, B, n, rng):
    """Logits of several shapes: N(0, s^2), U(-a, a), near-identity, a rank-one
    term plus noise, and the per-matrix scale mix of the hard workload."""
    if kind.startswith("normal"):
        return float(kind.split(":")[1]) * rng.standard_normal((B, n, n))
    if kind.startswith("unif"):
        a = float(kind.split(":")[1])
        return rng.uniform(-a, a, (B, n, n))
    if kind == "nearI":
        return 0.5 * rng.standard_normal((B, n, n)) + 2.0 * np.eye(n)
    if kind == "lowrank":
        return 3.0 * rng.standard_normal((B, n, 1)) * rng.standard_normal((B, 1, n)) \
            + 0.3 * rng.standard_normal((B, n, n))
    s = rng.choice([1.0, 3.0, 5.0, 8.0], size=(B, 1, 1))
    return s * rng.standard_normal((B, n, n))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("kind", SWEEP_KINDS)
def test_distribution_sweep(kind, n, io):
    """The one-launch forward + backward on logits of many shapes against the
    oracle: forward and residual gates as everywhere, the backward by
    backward_check (bf16: its part (a), with half an ulp for the stored rounding),
    and the forward-only launch equal to the one-launch forward bit for bit.
    In bf16 storage the residual is that of T rebuilt from the stored fp32 dual,
    whose own rounding at the |beta| ~ 40 of N(0, 10^2) logits check_forward
    allows for."""
    rng = np.random.default_rng([n, SWEEP_KINDS.index(kind), int(io == "bf16")])
    B = 3000 + 17 * n
    print("case sweep %s n=%d %s" % (kind, n, io), flush=True)
    H32 = sweep_logits(kind, B, n, rng).astype(np.float32)
    G32 = rng.standard_normal((B, n, n)).astype(np.float32)
    w = W.Workload(key="sweep", title=kind, B=B, n=n, io=io, logits=None, upstream=None, passes="fwd+bwd",
                   seed=0, max_iter=100)
    Hs = W.f32_to_bf16_bits(H32) if io == "bf16" else H32
    Gs = W.f32_to_bf16_bits(G32) if io == "bf16" else G32
    H, G = as_storage(Hs, w), as_storage(Gs, w)
    T, dH = torch.empty_like(H), torch.empty_like(H)
    dual = torch.empty((B, n), device=DEV)
    fused = bp.birkhoff_fwd_bwd_bf16 if io == "bf16" else bp.birkhoff_fwd_bwd
    fused(H, G, T, dual, dH, w.tol, w.max_iter)
    _, T2, dual2, _ = run_fwd(w, Hs)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    H64, G64 = W.decode_f64(Hs), W.decode_f64(Gs)
    T_ref, _, st = oracle.project(H64, sk_cap=5_000)
    assert (st >= 0).all()
    check_forward(w, H64, host_f64(T), dual.cpu().numpy().astype(np.float64), T_ref)
    dHg = host_f64(dH)
    if io == "bf16":
        # backward_check's part (a) only: the kernel differentiates at its fp32
        # iterate, which is not stored (the stored T is rounded to bf16); T rebuilt
        # from (logits, dual) stands in for it, within 2e-6 of it (check_forward's
        # rebuilt-T distance on fp32 storage stays below that), which widens the
        # gate by 2(n-1) 2e-6 / lambda; and the stored dH is rounded once more, so
        # half an ulp per entry is taken off the error
        Tu = rebuilt_T(H64, host_f64(dual))
        ref = oracle.bwd(Tu, G64)
        dHg = ref + np.sign(dHg - ref) * np.maximum(np.abs(dHg - ref) - half_ulp_bf16(ref), 0.0)
        gt = np.abs(G64 * Tu).max(axis=(1, 2))
        gate = 1e-4 * np.abs(ref).max(axis=(1, 2)) + gt * (8 * n * U32 + colres(Tu) + 2 * (n - 1) * 2e-6) / np.maximum(
            delta_lambda_min(Tu), 1e-300)
        ratio = np.abs(dHg - ref).max(axis=(1, 2)) / gate
        assert (ratio <= 1.0).all(), ratio.max()
        print("  bwd worst error/gate %.2f" % ratio.max())
    else:
        loose, r = backward_check(dHg, host_f64(T), G64, T_ref, kind)
        print("  bwd worst error/gate %.2f, %d of %d with a loose gate" % (r, loose, B))


def test_binding_rejects_bad_arguments():
    """The binding's checks, and the C ABI's behind them, reject malformed calls
    before anything is launched; a good call still works afterwards."""
    B = 64
    H = torch.randn((B, 4, 4), device=DEV)
    T = torch.empty_like(H)
    dual = torch.empty((B, 4), device=DEV)
    with pytest.raises(ValueError):
        bp.birkhoff_fwd(H.cpu(), T, dual)                                  # host tensor
    with pytest.raises(TypeError):
        bp.birkhoff_fwd(H.double(), T, dual)                               # wrong dtype
    with pytest.raises(ValueError):
        bp.birkhoff_fwd(H.transpose(1, 2), T, dual)                        # not contiguous
    with pytest.raises(ValueError):
        bp.birkhoff_fwd(H[:, :, :3].contiguous(), T, dual)                 # not square
    with pytest.raises(ValueError):
        bp.birkhoff_fwd(H, torch.empty((B + 1, 4, 4), device=DEV), dual)  # T of another batch
    with pytest.raises(ValueError):
        bp.birkhoff_fwd(H, T, torch.empty((B, 3), device=DEV))             # dual of another shape
    with pytest.raises(bp.BirkhoffError) as e:
        bp.birkhoff_fwd(H, T, dual, tol=0.0)                               # tol must be positive
    assert e.value.code == -1
    with pytest.raises(bp.BirkhoffError) as e:
        H5 = torch.randn((B, 5, 5), device=DEV)
        bp.birkhoff_fwd(H5, torch.empty_like(H5), torch.empty((B, 5), device=DEV))   # n not 4 or 8
    assert e.value.code == -1
    base = torch.randn(B * 16 + 4, device=DEV)
    Hmis = base[1:1 + B * 16].view(B, 4, 4)                                 # 4 bytes past a 16-byte boundary
    assert Hmis.is_contiguous() and Hmis.data_ptr() % 16 == 4
    with pytest.raises(bp.BirkhoffError) as e:
        bp.birkhoff_fwd(Hmis, T, dual)
    assert e.value.code == -2
    bp.birkhoff_fwd(H, T, dual)
    torch.cuda.synchronize()
    assert residual(host_f64(T)).max() <= RES_TOL


# ------------------------------------------ large logit spans and underflow

@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("sigma", [16.0, 20.0, 30.0])
def test_large_logit_spans(sigma, n):
    """Logits N(0, sigma^2), beyond the pages' largest scale (10): spans reach 170,
    so the starting row softmaxes have entries that underflow fp32, while the
    iteration forms T multiplicatively.  Every matrix either converges -- and then
    meets the forward gates against the oracle, equals the T rebuilt from its dual
    and passes backward_check -- or reports -1, exactly where the float64 column
    residual of its T exceeds tol/2 (the kernel decides in fp32).  The float64
    oracle cannot certify a handful of the largest-scale matrices; those are
    checked by eq (1)'s optimality conditions only (T = D1 exp(H) D2 with the
    returned dual, marginals to 1e-5), and their number is bounded."""
    B = 4096 + 19
    rng = np.random.default_rng([int(sigma), n, 11])
    H32 = (sigma * rng.standard_normal((B, n, n))).astype(np.float32)
    G32 = rng.standard_normal((B, n, n)).astype(np.float32)
    w = W.Workload(key="spans", title="N(0,%g^2)" % sigma, B=B, n=n, io="f32", logits=None, upstream=None,
                   passes="fwd+bwd", seed=0, max_iter=100)
    print("case spans sigma=%g n=%d" % (sigma, n), flush=True)
    H, T, dual, (iters, fb) = run_fwd(w, H32, stats=True)
    _, _, T2, dual2, dH = run_fused(w, H32, G32)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    H64, G64 = H32.astype(np.float64), G32.astype(np.float64)
    Tg, dg = host_f64(T), host_f64(dual)
    it, fbn = iters.cpu().numpy(), fb.cpu().numpy()
    conv = it >= 0
    assert conv.mean() >= 0.99
    assert ((fbn >= 0) & (fbn <= np.where(conv, it, w.max_iter))).all()
    assert np.isfinite(Tg).all()
    # eq (1)'s optimality conditions for every converged matrix
    assert residual(Tg)[conv].max() <= RES_TOL
    assert np.abs(Tg - rebuilt_T(H64, dg)).max(axis=(1, 2))[conv].max() <= FWD_TOL
    # -1 exactly where tol is not met
    assert (colres(Tg)[~conv] > 0.5 * w.tol).all()
    T_ref, _, st = oracle.project(H64, sk_cap=5_000)
    cert = st >= 0
    assert (~cert).sum() <= B // 200, (~cert).sum()
    sel = conv & cert
    err = np.abs(Tg - T_ref).max(axis=(1, 2))
    assert err[sel].max() <= FWD_TOL, err[sel].max()
    loose, r = backward_check(host_f64(dH)[sel], Tg[sel], G64[sel], T_ref[sel], "fused")
    print("  unconverged %d, uncertified %d, fallback matrices %d, max updates %d, fwd err %.2e, "
          "bwd worst error/gate %.2f (%d loose)" % ((~conv).sum(), (~cert).sum(), (fbn > 0).sum(), it.max(),
                                                    err[sel].max(), r, loose))


def underflow_batch(n, depth, B=256, seed=12):
    """Logits whose starting row softmaxes lose entries that matter: rows 0 and 1
    put `depth` in column 0 (so the projection must share column 0 between them,
    and the dual pushes column 0 down by about depth), and hold 0 or -10 in the
    other columns, whose entries at beta = 0 are e^-depth and e^-(depth + 10)
    relative to the row: subnormal or zero in fp32 for depth >= 88.  In the
    projection those entries carry about half of rows 0 and 1.  The other rows
    are N(0, 1).  Each matrix gets its own random row and column order."""
    rng = np.random.default_rng([n, int(depth), seed])
    out = np.empty((B, n, n), dtype=np.float32)
    for b in range(B):
        H = rng.standard_normal((n, n))
        H[0] = 0.0
        H[1] = 0.0
        H[0, 0] = H[1, 0] = depth
        H[0, 1] = H[1, 2] = -10.0
        out[b] = H[rng.permutation(n)][:, rng.permutation(n)]
    return out


@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("depth", [60.0, 88.0, 95.0, 103.0, 120.0])
def test_underflowed_start_is_verified(n, depth):
    """underflow_batch: the starting T has lost entries (zero or subnormal), so these
    lanes rebuild T from the logits at their dual when they converge and go on from
    it.  Every matrix must converge to the oracle's projection, through the
    forward (statistics variant and plain), the one-launch forward + backward and
    the gathering path alike.  The step rule needs many updates here: while rows 0
    and 1 both sit on column 0 the gradient norm does not decrease, no step size
    is accepted, and each fallback sweep moves the dual by about log 2 -- so the
    cap is 1000 updates."""
    Hs = underflow_batch(n, depth)
    B = Hs.shape[0]
    w = W.Workload(key="underflow", title="", B=B, n=n, io="f32", logits=None, upstream=None, passes="fwd+bwd",
                   seed=0, max_iter=1000)
    print("case underflow n=%d depth=%g" % (n, depth), flush=True)
    H, T, dual, (iters, fb) = run_fwd(w, Hs, stats=True)
    _, T3, dual3, _ = run_fwd(w, Hs)
    G32 = np.random.default_rng(5).standard_normal(Hs.shape).astype(np.float32)
    _, _, T2, dual2, dH = run_fused(w, Hs, G32)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, dual2) and torch.equal(T, T3) and torch.equal(dual, dual3)
    it, fbn = iters.cpu().numpy(), fb.cpu().numpy()
    assert (it >= 0).all(), (it < 0).sum()
    assert ((fbn >= 0) & (fbn <= it)).all()
    # the shared column keeps every step size from being accepted: these
    # matrices converge through fallback sweeps, and meet the gates below
    assert (fbn > 0).mean() >= 0.5, (fbn > 0).mean()
    print("  updates: mean %.1f max %d, fallback sweeps max %d" % (it.mean(), it.max(), fbn.max()))
    H64 = Hs.astype(np.float64)
    T_ref, _, st = oracle.project(H64, sk_cap=5_000)
    assert (st >= 0).all()
    Tg = host_f64(T)
    check_forward(w, H64, Tg, host_f64(dual), T_ref)
    # the lost entries matter: some matrix has an entry of T_ref above 0.1 whose
    # starting value in fp32 was below 2^-100
    U = H64 - H64.max(axis=2, keepdims=True)
    assert ((U < -100 * np.log(2)) & (T_ref > 0.1)).any() or depth < 88
    backward_check(host_f64(dH), Tg, G32.astype(np.float64), T_ref, "fused")


# ------------------------------------------- degenerate eq (13) systems

def permutation_logits(n, c, B=64, seed=3):
    """c times a random permutation matrix per matrix, plus N(0, 0.25^2): for large
    c the projection is within e^-c of the permutation (exactly it, in fp32, for c
    beyond about 104), where Delta is numerically singular or zero."""
    rng = np.random.default_rng([n, int(c), seed])
    H = 0.25 * rng.standard_normal((B, n, n))
    for b in range(B):
        H[b, np.arange(n), rng.permutation(n)] += c
    return H.astype(np.float32)


@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("c", [30.0, 40.0, 60.0, 120.0])
def test_backward_near_permutations(n, c):
    """eq (13) where Delta is numerically singular: dH, whose exact value is within
    O(e^-c |G|) of zero (T is locally constant at a permutation), stays finite and
    below 1e-6 |G| through every backward entry point -- the dual-based backward,
    the one from T, the one-launch forward + backward and autograd -- and is
    exactly zero once T is an exact permutation in fp32."""
    Hs = permutation_logits(n, c)
    B = Hs.shape[0]
    G32 = np.random.default_rng([n, int(c)]).standard_normal(Hs.shape).astype(np.float32)
    H, G = dev(Hs), dev(G32)
    print("case permutation n=%d c=%g" % (n, c), flush=True)
    T, dual, dH1 = bp.project_fwd_bwd(H, G)
    dH2 = bp.project_bwd(H, dual, G)
    dH3 = torch.empty_like(G)
    bp.birkhoff_bwd_from_T(T, G, dH3)
    Ha = H.clone().requires_grad_(True)
    (bp.BirkhoffProjection.apply(Ha) * G).sum().backward()
    torch.cuda.synchronize()
    gmax = np.abs(G32).max()
    Tg = host_f64(T)
    exact = bool(((Tg == 0.0) | (Tg == 1.0)).all())
    for name, d in (("fused", dH1), ("bwd", dH2), ("from_T", dH3), ("autograd", Ha.grad)):
        dh = host_f64(d)
        assert np.isfinite(dh).all(), name
        assert np.abs(dh).max() <= 1e-6 * gmax, (name, np.abs(dh).max())
        if exact:
            assert (dh == 0.0).all(), name
    print("  T exact permutation: %s; max|dH| %.2e |G|" % (exact, np.abs(host_f64(dH1)).max() / gmax))


@pytest.mark.parametrize("n", [4, 8])
def test_backward_deflated_block(n):
    """A matrix with one dominant logit (H_00 = 200, spread over the same rows and
    columns elsewhere N(0, 1)) projects onto diag(1, T') up to e^-100, with T' the
    projection of the trailing (n-1) x (n-1) block; its gradient is diag(0, dH')
    with dH' eq (13) for that block.  The smaller problem is solved by the oracle
    on its own, so the n x n kernels are pinned to an (n-1) x (n-1) reference, in
    a case where the n x n Delta has a zero row and column."""
    rng = np.random.default_rng([n, 77])
    B = 512
    Hs = rng.standard_normal((B, n, n)).astype(np.float32)
    Hs[:, 0, 0] = 200.0
    G32 = rng.standard_normal((B, n, n)).astype(np.float32)
    H, G = dev(Hs), dev(G32)
    print("case deflated n=%d" % n, flush=True)
    T, dual, dH = bp.project_fwd_bwd(H, G, max_iter=100)
    dH2 = torch.empty_like(G)
    bp.birkhoff_bwd_from_T(T, G, dH2)
    torch.cuda.synchronize()
    Ts, _, st = oracle.project(Hs[:, 1:, 1:].astype(np.float64))
    assert (st >= 0).all()
    dHs = oracle.bwd(Ts, G32[:, 1:, 1:].astype(np.float64))
    Tg = host_f64(T)
    assert np.abs(Tg[:, 0, 0] - 1.0).max() <= FWD_TOL
    assert np.abs(Tg[:, 0, 1:]).max() <= FWD_TOL and np.abs(Tg[:, 1:, 0]).max() <= FWD_TOL
    assert np.abs(Tg[:, 1:, 1:] - Ts).max() <= FWD_TOL
    # backward_check's gate (b) for the block: its T is within d of T' (the
    # leakage into row and column 0 stops at the forward's tol)
    Gb = G32[:, 1:, 1:].astype(np.float64)
    gt = np.abs(Gb * Ts).max(axis=(1, 2))
    d = np.abs(Tg[:, 1:, 1:] - Ts).max(axis=(1, 2))
    gate = (BWD_TOL * np.abs(dHs).max(axis=(1, 2)) + 2 * np.abs(Gb).max(axis=(1, 2)) * d
            + gt * (8 * n * U32 + colres(Tg) + 2 * (n - 1) * d) / delta_lambda_min(Ts))
    for name, dd in (("fused", dH), ("from_T", dH2)):
        dh = host_f64(dd)
        assert np.abs(dh[:, 0, :]).max() <= 1e-6 * np.abs(G32).max(), name
        assert np.abs(dh[:, :, 0]).max() <= 1e-6 * np.abs(G32).max(), name
        err = np.abs(dh[:, 1:, 1:] - dHs).max(axis=(1, 2))
        assert (err <= gate).all(), (name, (err / gate).max())
    print("  block error/gate %.2f" % (np.abs(host_f64(dH)[:, 1:, 1:] - dHs).max(axis=(1, 2)) / gate).max())


@pytest.mark.parametrize("n", [4, 8])
def test_results_do_not_depend_on_the_batch(n):
    """A matrix's T and dual do not depend on the other matrices of the batch or
    on its position in it: the start's extra sweeps and the convergence check are
    each lane's own decisions, and a gathered matrix goes through the same updates
    wherever it is carried on.  Logits of mixed scales (N(0, s^2), s from 0.5 to
    12) are projected as one batch, in reverse order, and in sub-batches of 1, 63
    and 200; every result must equal the first bit for bit (gathering forward and
    fused kernel alike)."""
    rng = np.random.default_rng([n, 77])
    B = 1000
    scales = rng.choice([0.5, 1.0, 3.0, 8.0, 12.0], size=B)
    H32 = (scales[:, None, None] * rng.standard_normal((B, n, n))).astype(np.float32)
    G32 = rng.standard_normal((B, n, n)).astype(np.float32)
    w = W.Workload(key="batch", title="", B=B, n=n, io="f32", logits=None, upstream=None, passes="fwd+bwd",
                   seed=0, max_iter=100)
    print("case batch independence n=%d" % n, flush=True)
    _, T, dual, _ = run_fwd(w, H32)
    _, _, T2, dual2, _ = run_fused(w, H32, G32)
    torch.cuda.synchronize()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    Tn, dn = T.cpu().numpy(), dual.cpu().numpy()
    rev = np.arange(B)[::-1]
    _, Tr, dr, _ = run_fwd(w, H32[rev])
    torch.cuda.synchronize()
    assert np.array_equal(Tr.cpu().numpy(), Tn[rev]) and np.array_equal(dr.cpu().numpy(), dn[rev])
    for lo, hi in ((137, 138), (500, 563), (800, 1000)):
        _, Ts, ds, _ = run_fwd(w, H32[lo:hi])
        _, _, Tf, df, _ = run_fused(w, H32[lo:hi], G32[lo:hi])
        torch.cuda.synchronize()
        for X, Y in ((Ts, T), (Tf, T)):
            assert np.array_equal(X.cpu().numpy(), Y.cpu().numpy()[lo:hi]), (lo, hi)
        for X in (ds, df):
            assert np.array_equal(X.cpu().numpy(), dn[lo:hi]), (lo, hi)


def test_double_backward_raises():
    """The autograd functions' backward passes are computed by the kernels, not
    from differentiable torch operations, so a second derivative through them is
    refused rather than silently zero."""
    H = torch.randn((64, 4, 4), device=DEV, requires_grad=True)
    T = bp.BirkhoffProjection.apply(H)
    (g,) = torch.autograd.grad((T * T).sum(), H, create_graph=True)
    with pytest.raises(RuntimeError):
        g.sum().backward()
    # the general plan (uniform marginals of mass one) and the fused mixing
    cost = torch.randn((64, 4, 6), device=DEV, requires_grad=True)
    a = torch.full((64, 4), 0.25, device=DEV)
    b = torch.full((64, 6), 1.0 / 6.0, device=DEV)
    P = bp.EntropicOT.apply(cost, a, b, 1.0)
    (g,) = torch.autograd.grad((P * P).sum(), cost, create_graph=True)
    with pytest.raises(RuntimeError):
        g.sum().backward()
    Hm = torch.randn((8, 4, 4), device=DEV, requires_grad=True)
    x = torch.randn((8, 4, 64), device=DEV, requires_grad=True)
    y = bp.ProjectMix.apply(Hm, x)
    gH, gx = torch.autograd.grad((y * y).sum(), (Hm, x), create_graph=True)
    with pytest.raises(RuntimeError):
        (gH.sum() + gx.sum()).backward()
