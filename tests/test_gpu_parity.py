"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded inputs.  Needs an MI355X; run with -m gpu.

Gates (fp32 storage):
  forward   max |T - T_ref| <= 1e-5 over every entry;
  residual  max(|rowsum - 1|, |colsum - 1|) of the GPU's T, summed in float64, <= 1e-5;
  backward  per matrix max|dH - dH_ref| / max|dH_ref| <= 1e-4.
bf16 storage adds half a bf16 ulp of the reference value to the T and dH gates
(an fp32-exact answer must still be rounded once to be stored), and takes the
residual on T rebuilt in float64 from the logits and the fp32 dual.
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
    B, n = Hs.shape[0], w.n
    H = as_storage(Hs, w)
    T = torch.empty_like(H)
    dual = torch.empty((B, n), dtype=torch.float32, device=DEV)
    iters = None
    if w.io == "bf16":
        bp.birkhoff_fwd_bf16(H, T, dual, w.tol, w.max_iter)
    elif stats:
        iters = torch.empty(B, dtype=torch.int32, device=DEV)
        bp.birkhoff_fwd_ex(H, T, dual, iters, w.tol, w.max_iter)
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
        res = residual(rebuilt_T(H64, dual_gpu)).max()
    else:
        assert err.max() <= FWD_TOL, err.max()
        res = residual(T_gpu).max()
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
    H, T, dual, _ = run_fwd(w, Hs)
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
        # the layout is the intended one: slow matrices need more than 4 updates in fp32
        assert (it >= 0).all()
        np.testing.assert_array_equal(it > 4, want_slow)
        T_ref, _, st = oracle.project(Hs.astype(np.float64))
        assert (st >= 0).all()
        check_forward(W.WORKLOADS["hard"], Hs.astype(np.float64), host_f64(T), None, T_ref)
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

def conditioned_backward_check(dH_gpu, dH_ref, T_ref):
    """Backward gate on inputs whose projection is close to a permutation.  dH
    depends on T through Delta^{-1} (eq 13), Delta = I - T_{-n}^T T_{-n}: an
    entrywise change d of T changes each entry of Delta by at most 2d (columns of
    T sum to one), so ||dDelta||_2 <= ||dDelta||_F <= 2(n-1)d (6d for n = 4), and
    dH moves by up to 2(n-1)d / lambda_min(Delta) relative to its size to first
    order.  With d the forward tolerance 1e-5 (the fp32 T, which the backward
    starts from, is only that close to T_ref), the per-matrix gate is
    1e-4 + 2(n-1)e-5 / lambda_min."""
    Tm = T_ref[:, :, :-1]
    n1 = Tm.shape[2]
    Delta = np.eye(n1)[None] - np.matmul(Tm.transpose(0, 2, 1), Tm)
    lam = np.linalg.eigvalsh(Delta)[:, 0]
    scale = np.abs(dH_ref).max(axis=(1, 2))
    rel = np.abs(dH_gpu - dH_ref).max(axis=(1, 2)) / scale
    bound = BWD_TOL + 2 * n1 * FWD_TOL / np.maximum(lam, 1e-300)
    assert (rel <= bound).all(), "worst excess %.3e (lambda_min %.3e)" % (
        (rel / bound).max(), lam[np.argmax(rel / bound)])
    return float(rel.max()), float((rel[lam > 0.1]).max(initial=0.0))


@pytest.mark.parametrize("B", [512, 8192])
def test_parity_pages_timing_shape(B):
    """The pages' timing inputs (4x4, N(0, 10^2) logits: farther from uniform than any
    benchmark workload) through the forward (gathering kernel), the backward and the
    one-launch forward + backward, against the oracle.  Many of these projections are
    nearly permutations, where the backward is ill-conditioned (the smallest
    eigenvalue of Delta goes down to 1e-11), so its gate widens with the condition
    of Delta (conditioned_backward_check)."""
    w = W.pages_shape_workload(B)
    print("case pages shape", B, flush=True)
    Hs = W.make_logits(w)
    Gs = W.make_upstream(w)
    H64 = Hs.astype(np.float64)
    H, T, dual, iters = run_fwd(w, Hs, stats=True)
    dH = run_bwd(w, H, dual, Gs)
    _, _, T2, dual2, dH2 = run_fused(w, Hs, Gs)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    assert (it >= 0).all(), (it < 0).sum()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    err, res = check_forward(w, H64, host_f64(T), None, T_ref)
    dH_ref = oracle.bwd(T_ref, Gs.astype(np.float64))
    rel, rel_wc = conditioned_backward_check(host_f64(dH), dH_ref, T_ref)
    rel2, rel2_wc = conditioned_backward_check(host_f64(dH2), dH_ref, T_ref)
    print("  max updates %d, fwd err %.2e, residual %.2e, bwd rel %.2e / fused %.2e "
          "(where lambda_min > 0.1: %.2e / %.2e)" % (it.max(), err, res, rel, rel2, rel_wc, rel2_wc))


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
    check_forward(W.WORKLOADS["hard"], Hs.astype(np.float64), host_f64(T), None, T_ref)


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
    backward against the oracle (backward gate as conditioned_backward_check)."""
    w = W.Workload(key="n8_sigma_mix", title="8x8 fp32, H~N(0,s^2), s per matrix from {1,3,5,8}",
                   B=4096 + 19, n=8, io="f32", logits=("sigma_mix", (1.0, 3.0, 5.0, 8.0)),
                   upstream=("normal", 1.0), passes="fwd+bwd", seed=9, max_iter=100, sk_cap=5_000)
    print("case n8 large logits", flush=True)
    Hs, Gs = W.make_logits(w), W.make_upstream(w)
    H64 = Hs.astype(np.float64)
    H, T, dual, iters = run_fwd(w, Hs, stats=True)
    dH = run_bwd(w, H, dual, Gs)
    _, _, T2, dual2, dH2 = run_fused(w, Hs, Gs)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    assert (it >= 0).all(), (it < 0).sum()
    assert torch.equal(T, T2) and torch.equal(dual, dual2)
    T_ref, _, st = oracle.project(H64, sk_cap=w.sk_cap)
    assert (st >= 0).all()
    err, res = check_forward(w, H64, host_f64(T), None, T_ref)
    dH_ref = oracle.bwd(T_ref, Gs.astype(np.float64))
    rel, rel_wc = conditioned_backward_check(host_f64(dH), dH_ref, T_ref)
    rel2, rel2_wc = conditioned_backward_check(host_f64(dH2), dH_ref, T_ref)
    print("  max updates %d, fwd err %.2e, residual %.2e, bwd rel %.2e / fused %.2e "
          "(where lambda_min > 0.1: %.2e / %.2e)" % (it.max(), err, res, rel, rel2, rel_wc, rel2_wc))


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
    oracle: forward and residual gates as everywhere, the backward gate widened
    with the condition of Delta (conditioned_backward_check, bf16 adding half an
    ulp), and the forward-only launch equal to the one-launch forward bit for bit.
    bf16 storage stops at scale 8: at N(0, 10^2) the fp32 dual, |beta| ~ 30, is
    itself rounded by ~2e-6, so T rebuilt from it misses the 1e-5 residual gate."""
    if io == "bf16" and kind == "normal:10":
        pytest.skip("outside the bf16 reading's residual gate (see docstring)")
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
    dH_ref = oracle.bwd(T_ref, G64)
    dHg = host_f64(dH)
    if io == "bf16":   # the stored dH is rounded once more: half an ulp of slack per entry
        dHg = dH_ref + np.sign(dHg - dH_ref) * np.maximum(np.abs(dHg - dH_ref) - half_ulp_bf16(dH_ref), 0.0)
    rel, rel_wc = conditioned_backward_check(dHg, dH_ref, T_ref)
    print("  bwd rel %.2e (where lambda_min > 0.1: %.2e)" % (rel, rel_wc))


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
