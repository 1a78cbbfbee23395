"""GPU parity for the projection fused with its mHC consumer (birkhoff_fwd_mix /
birkhoff_mix_bwd and their bf16 variants, through the C ABI) against the float64
oracle on the same seeded inputs.  Needs an MI355X; run with -m gpu.

Gates:
  T, dual   bit-identical to birkhoff_fwd on the same logits (same iteration);
  y = T x   |y - y_ref| <= 4e-5 max_j |x_jc| per column c: y_ic = sum_j T_ij x_jc, and each
            T_ij is within the forward gate 1e-5 of the reference; bf16 storage adds half
            a bf16 ulp of y_ref (one rounding of the stored result);
  dx = T^T dy  the same bound with dy;
  dH        per token max|dH - dH_ref| / max(max|dH_ref|, 0.04 max|dT_ref o T_ref|) <= 1e-4,
            dH_ref = eq (13) at the reference plan of dT_ref = dy x^T (the floor as for the
            general-OT backward: dH sums terms of that size, which can cancel).
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
BWD_TOL = 1e-4


def workload(io, C, seed=80):
    return W.MixWorkload(key="mix_t", title="test", B=0, C=C, io=io, logits=("near_identity", 0.5, 2.0),
                         hidden=("normal", 1.0), upstream=("normal", 1.0), seed=seed)


def dev(a, io="f32"):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.view(torch.bfloat16) if io == "bf16" else t


def f64(t):
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy().astype(np.float64)


def half_ulp_bf16(v):
    av = np.abs(v)
    e = np.floor(np.log2(np.where(av > 0, av, 1.0)))
    return np.where(av > 0, 2.0 ** (e - 8), 0.0)


def check_streams(out, ref, src, io):
    bound = 4 * FWD_TOL * np.abs(src).max(axis=1, keepdims=True)
    if io == "bf16":
        bound = bound + half_ulp_bf16(ref)
    err = np.abs(out - ref) - bound
    assert err.max() <= 0, "worst excess %.3e" % err.max()


def run_forward(H, x, io):
    T, dual, y = bp.project_mix(dev(H), dev(x, io))
    T0 = torch.empty_like(T)
    d0 = torch.empty_like(dual)
    bp.birkhoff_fwd(dev(H), T0, d0)
    torch.cuda.synchronize()
    assert torch.equal(T, T0) and torch.equal(dual, d0)
    return T, dual, y


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,C", [(1, 8), (63, 64), (64, 520), (65, 8), (300, 256), (200, 4096)])
def test_forward_mix(io, B, C):
    w = workload(io, C)
    H, x, _ = W.make_mix(w, B=B)
    print("mix fwd io=%s B=%d C=%d" % (io, B, C), flush=True)
    T, dual, y = run_forward(H, x, io)
    T_ref, _, st = oracle.project(H.astype(np.float64))
    assert (st >= 0).all()
    assert np.abs(f64(T) - T_ref).max() <= FWD_TOL
    xd = W.decode_f64(x)
    check_streams(f64(y), oracle.mix(T_ref, xd), xd, io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,C", [(1, 8), (63, 64), (65, 520), (300, 256), (130, 4096)])
def test_backward_mix(io, B, C):
    w = workload(io, C, seed=81)
    H, x, dy = W.make_mix(w, B=B)
    print("mix bwd io=%s B=%d C=%d" % (io, B, C), flush=True)
    T, _, _ = bp.project_mix(dev(H), dev(x, io))
    dH, dx = bp.project_mix_bwd(T, dev(x, io), dev(dy, io))
    torch.cuda.synchronize()
    T_ref, _, _ = oracle.project(H.astype(np.float64))
    xd, dyd = W.decode_f64(x), W.decode_f64(dy)
    dx_ref, dT_ref = oracle.mix_bwd(T_ref, xd, dyd)
    check_streams(f64(dx), dx_ref, dyd, io)
    dH_ref = oracle.bwd(T_ref, dT_ref)
    scale = np.maximum(np.abs(dH_ref).max(axis=(1, 2)), 0.04 * np.abs(dT_ref * T_ref).max(axis=(1, 2)))
    rel = np.abs(f64(dH) - dH_ref).max(axis=(1, 2)) / scale
    assert rel.max() <= BWD_TOL, "worst relative dH error %.3e" % rel.max()


def test_autograd_function():
    w = workload("f32", 64, seed=82)
    H, x, dy = W.make_mix(w, B=100)
    Hd = dev(H).requires_grad_(True)
    xd = dev(x).requires_grad_(True)
    y = bp.ProjectMix.apply(Hd, xd)
    (y * dev(dy)).sum().backward()
    torch.cuda.synchronize()
    T_ref, _, _ = oracle.project(H.astype(np.float64))
    x64, dy64 = x.astype(np.float64), dy.astype(np.float64)
    check_streams(f64(y.detach()), oracle.mix(T_ref, x64), x64, "f32")
    dx_ref, dT_ref = oracle.mix_bwd(T_ref, x64, dy64)
    check_streams(f64(xd.grad), dx_ref, dy64, "f32")
    dH_ref = oracle.bwd(T_ref, dT_ref)
    rel = np.abs(f64(Hd.grad) - dH_ref).max(axis=(1, 2)) / np.abs(dH_ref).max(axis=(1, 2))
    assert rel.max() <= BWD_TOL


def test_doubly_stochastic_mixing_conserves_stream_sums():
    """Columns of T sum to one, so each column of y keeps the sum over the streams."""
    w = workload("f32", 512, seed=83)
    H, x, _ = W.make_mix(w, B=256)
    _, _, y = run_forward(H, x, "f32")
    ys = f64(y).sum(1)
    xs = x.astype(np.float64).sum(1)
    assert np.abs(ys - xs).max() <= 4e-5 * np.abs(x).max()


def test_zero_features_projects_only():
    w = workload("f32", 8, seed=84)
    H, _, _ = W.make_mix(w, B=100)
    x = torch.empty((100, 4, 0), dtype=torch.float32, device=DEV)
    T, dual, y = bp.project_mix(dev(H), x)
    dH, dx = bp.project_mix_bwd(T, x, torch.empty_like(x))
    torch.cuda.synchronize()
    assert y.shape == (100, 4, 0) and dx.shape == (100, 4, 0)
    T_ref, _, _ = oracle.project(H.astype(np.float64))
    assert np.abs(f64(T) - T_ref).max() <= FWD_TOL
    # dT = 0, so dH = 0
    assert float(dH.abs().max()) == 0.0


def test_empty_batch():
    H = torch.empty((0, 4, 4), dtype=torch.float32, device=DEV)
    x = torch.empty((0, 4, 16), dtype=torch.float32, device=DEV)
    T, dual, y = bp.project_mix(H, x)
    dH, dx = bp.project_mix_bwd(T, x, torch.empty_like(x))
    torch.cuda.synchronize()
    assert y.shape == (0, 4, 16) and dH.shape == (0, 4, 4)


def test_full_size_workload_sampled():
    """The benchmark workload at its full size and launch configuration: a seeded
    sample of 128 tokens is compared with the oracle one by one."""
    w = W.MIX_WORKLOADS["mix"]
    H, x, dy = W.make_mix(w)
    print("mix full size B=%d C=%d" % (w.B, w.C), flush=True)
    xd, dyd = dev(x, w.io), dev(dy, w.io)
    T, dual, y = bp.project_mix(dev(H), xd)
    dH, dx = bp.project_mix_bwd(T, xd, dyd)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(85).choice(w.B, 128, replace=False))
    it = torch.from_numpy(idx).to(DEV)
    T_ref, _, st = oracle.project(H[idx].astype(np.float64))
    assert (st >= 0).all()
    assert np.abs(f64(T[it]) - T_ref).max() <= FWD_TOL
    xs, dys = W.decode_f64(x[idx]), W.decode_f64(dy[idx])
    check_streams(f64(y[it]), oracle.mix(T_ref, xs), xs, w.io)
    dx_ref, dT_ref = oracle.mix_bwd(T_ref, xs, dys)
    check_streams(f64(dx[it]), dx_ref, dys, w.io)
    dH_ref = oracle.bwd(T_ref, dT_ref)
    scale = np.maximum(np.abs(dH_ref).max(axis=(1, 2)), 0.04 * np.abs(dT_ref * T_ref).max(axis=(1, 2)))
    assert (np.abs(f64(dH[it]) - dH_ref).max(axis=(1, 2)) / scale).max() <= BWD_TOL


def test_streams_beyond_32bit_offsets():
    """140,000 tokens of 4 x 4096 bf16 hidden states: each stream array is 4.6 GB,
    so byte offsets pass 2^32 (the benchmark workload stays at 2.1 GB).  Inputs
    are drawn on the device; a sample of tokens that includes the last ones is
    compared with the oracle."""
    B, C = 140_000, 4096
    print("mix 64-bit offsets B=%d C=%d" % (B, C), flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(91)
    H = torch.randn((B, 4, 4), generator=g, device=DEV) * 0.5 + 2.0 * torch.eye(4, device=DEV)
    x = torch.randn((B, 4, C), generator=g, device=DEV, dtype=torch.bfloat16)
    dy = torch.randn((B, 4, C), generator=g, device=DEV, dtype=torch.bfloat16)
    T, dual, y = bp.project_mix(H, x)
    dH, dx = bp.project_mix_bwd(T, x, dy)
    torch.cuda.synchronize()
    rng = np.random.default_rng(92)
    idx = np.unique(np.concatenate([np.arange(B - 16, B), rng.choice(B, 48, replace=False)]))
    it = torch.from_numpy(idx).to(DEV)
    H64 = f64(H[it])
    T_ref, _, st = oracle.project(H64)
    assert (st >= 0).all()
    assert np.abs(f64(T[it]) - T_ref).max() <= FWD_TOL
    xs, dys = f64(x[it]), f64(dy[it])
    check_streams(f64(y[it]), oracle.mix(T_ref, xs), xs, "bf16")
    dx_ref, dT_ref = oracle.mix_bwd(T_ref, xs, dys)
    check_streams(f64(dx[it]), dx_ref, dys, "bf16")
    dH_ref = oracle.bwd(T_ref, dT_ref)
    scale = np.maximum(np.abs(dH_ref).max(axis=(1, 2)), 0.04 * np.abs(dT_ref * T_ref).max(axis=(1, 2)))
    assert (np.abs(f64(dH[it]) - dH_ref).max(axis=(1, 2)) / scale).max() <= BWD_TOL
    del x, dy, y, dx
    torch.cuda.empty_cache()
