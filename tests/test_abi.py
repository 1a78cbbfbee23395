"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import math
import pathlib
import re

import pytest

import birkhoff_projection_amd as bp

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "birkhoff.h"

EINVAL, EALIGN = -1, -2


def declared_symbols():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not bp.library_path().exists():
        from birkhoff_projection_amd import build
        build.build()
    return bp.load_library()


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for n in ("birkhoff_fwd", "birkhoff_fwd_ex", "birkhoff_bwd", "sinkhorn_fwd",
              "birkhoff_fwd_bf16", "birkhoff_bwd_bf16", "birkhoff_fwd_bwd", "birkhoff_fwd_bwd_bf16",
              "birkhoff_bwd_from_T", "birkhoff_eot_fwd", "birkhoff_eot_bwd",
              "birkhoff_fwd_mix", "birkhoff_fwd_mix_bf16", "birkhoff_mix_bwd", "birkhoff_mix_bwd_bf16",
              "birkhoff_strerror", "birkhoff_abi_version", "birkhoff_clock_probe"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert bp.birkhoff_abi_version() == 2
    for code in (0, -1, -2, -3, 12345):
        s = bp.birkhoff_strerror(code)
        assert isinstance(s, str) and s


A = 1 << 20          # fake, 16-byte aligned addresses: never dereferenced on a rejected call
P = [A, A + 4096, A + 8192, A + 12288]


def fwd(lib, *a):
    return lib.birkhoff_fwd(*a)


@pytest.mark.parametrize("B,n,tol,it,want", [
    (-1, 4, 1e-6, 50, EINVAL),
    (5, 3, 1e-6, 50, EINVAL),
    (5, 16, 1e-6, 50, EINVAL),
    (5, 4, 0.0, 50, EINVAL),
    (5, 4, -1.0, 50, EINVAL),
    (5, 4, math.nan, 50, EINVAL),
    (5, 4, math.inf, 50, EINVAL),
    (5, 4, 1e-6, 0, EINVAL),
    (1 << 50, 4, 1e-6, 50, EINVAL),
    (0, 4, 1e-6, 50, 0),
])
def test_forward_argument_checks(lib, B, n, tol, it, want):
    assert lib.birkhoff_fwd(P[0], P[1], P[2], B, n, tol, it, None) == want
    assert lib.birkhoff_fwd_bf16(P[0], P[1], P[2], B, n, tol, it, None) == want
    assert lib.birkhoff_fwd_ex(P[0], P[1], P[2], P[3], None, B, n, tol, it, None) == want
    assert lib.birkhoff_fwd_ex(P[0], P[1], P[2], P[3], P[3] + 64, B, n, tol, it, None) == want


def test_null_and_misaligned_pointers(lib):
    B, n = 7, 4
    for k in range(3):
        ptrs = list(P[:3])
        ptrs[k] = None
        assert lib.birkhoff_fwd(*ptrs, B, n, 1e-6, 50, None) == EINVAL
        ptrs[k] = P[k] + 4
        assert lib.birkhoff_fwd(*ptrs, B, n, 1e-6, 50, None) == EALIGN
    assert lib.birkhoff_fwd_ex(P[0], P[1], P[2], None, None, B, n, 1e-6, 50, None) == EINVAL
    assert lib.birkhoff_fwd_ex(P[0], P[1], P[2], None, P[3], B, n, 1e-6, 50, None) == EINVAL
    assert lib.birkhoff_fwd_ex(P[0], P[1], P[2], P[3] + 2, None, B, n, 1e-6, 50, None) == EALIGN
    assert lib.birkhoff_fwd_ex(P[0], P[1], P[2], P[3], P[3] + 66, B, n, 1e-6, 50, None) == EALIGN
    for k in range(4):
        ptrs = list(P)
        ptrs[k] = None
        assert lib.birkhoff_bwd(*ptrs, B, n, None) == EINVAL
        assert lib.birkhoff_bwd_bf16(*ptrs, B, n, None) == EINVAL
        ptrs[k] = P[k] + 2
        assert lib.birkhoff_bwd(*ptrs, B, n, None) == EALIGN
    assert lib.sinkhorn_fwd(None, P[1], B, n, 20, None) == EINVAL
    assert lib.sinkhorn_fwd(P[0] + 4, P[1], B, n, 20, None) == EALIGN


@pytest.mark.parametrize("B,n,tol,it,want", [
    (-1, 4, 1e-6, 50, EINVAL),
    (5, 5, 1e-6, 50, EINVAL),
    (5, 4, 0.0, 50, EINVAL),
    (5, 4, math.nan, 50, EINVAL),
    (5, 4, 1e-6, 0, EINVAL),
    (0, 8, 1e-6, 50, 0),
])
def test_fused_argument_checks(lib, B, n, tol, it, want):
    Q = [A, A + 4096, A + 8192, A + 12288, A + 16384]
    assert lib.birkhoff_fwd_bwd(*Q, B, n, tol, it, None) == want
    assert lib.birkhoff_fwd_bwd_bf16(*Q, B, n, tol, it, None) == want


def test_fused_null_and_misaligned_pointers(lib):
    Q = [A, A + 4096, A + 8192, A + 12288, A + 16384]
    for k in range(5):
        ptrs = list(Q)
        ptrs[k] = None
        assert lib.birkhoff_fwd_bwd(*ptrs, 9, 4, 1e-6, 50, None) == EINVAL
        ptrs[k] = Q[k] + 8
        assert lib.birkhoff_fwd_bwd(*ptrs, 9, 4, 1e-6, 50, None) == EALIGN
        assert lib.birkhoff_fwd_bwd_bf16(*ptrs, 9, 8, 1e-6, 50, None) == EALIGN


def test_bwd_from_T_argument_checks(lib):
    assert lib.birkhoff_bwd_from_T(P[0], P[1], P[2], -1, 4, None) == EINVAL
    assert lib.birkhoff_bwd_from_T(P[0], P[1], P[2], 5, 6, None) == EINVAL
    assert lib.birkhoff_bwd_from_T(None, None, None, 0, 4, None) == 0
    for k in range(3):
        ptrs = list(P[:3])
        ptrs[k] = None
        assert lib.birkhoff_bwd_from_T(*ptrs, 5, 8, None) == EINVAL
        ptrs[k] = P[k] + 4
        assert lib.birkhoff_bwd_from_T(*ptrs, 5, 8, None) == EALIGN


def test_backward_and_sinkhorn_argument_checks(lib):
    assert lib.birkhoff_bwd(*P, -1, 4, None) == EINVAL
    assert lib.birkhoff_bwd(*P, 5, 5, None) == EINVAL
    assert lib.birkhoff_bwd(None, None, None, None, 0, 8, None) == 0
    assert lib.sinkhorn_fwd(P[0], P[1], 5, 4, 0, None) == EINVAL
    assert lib.sinkhorn_fwd(P[0], P[1], 5, 4, -3, None) == EINVAL
    assert lib.sinkhorn_fwd(P[0], P[1], 5, 7, 20, None) == EINVAL
    assert lib.sinkhorn_fwd(None, None, 0, 4, 20, None) == 0


# birkhoff_eot_fwd(cost, a, b, shared, T, dual, iters, B, n, m, eta, tol, max_iter, stream)
@pytest.mark.parametrize("B,n,m,eta,tol,it,want", [
    (-1, 4, 6, 0.5, 1e-6, 50, EINVAL),
    (5, 0, 6, 0.5, 1e-6, 50, EINVAL),
    (5, 9, 6, 0.5, 1e-6, 50, EINVAL),
    (5, 4, 1, 0.5, 1e-6, 50, EINVAL),
    (5, 4, 9, 0.5, 1e-6, 50, EINVAL),
    (5, 4, 6, 0.0, 1e-6, 50, EINVAL),
    (5, 4, 6, -1.0, 1e-6, 50, EINVAL),
    (5, 4, 6, math.nan, 1e-6, 50, EINVAL),
    (5, 4, 6, math.inf, 1e-6, 50, EINVAL),
    (5, 4, 6, 0.5, 0.0, 50, EINVAL),
    (5, 4, 6, 0.5, math.nan, 50, EINVAL),
    (5, 4, 6, 0.5, 1e-6, 0, EINVAL),
    (1 << 50, 4, 6, 0.5, 1e-6, 50, EINVAL),
    (0, 1, 2, 0.5, 1e-6, 50, 0),
    (0, 8, 8, 0.5, 1e-6, 50, 0),
])
def test_eot_forward_argument_checks(lib, B, n, m, eta, tol, it, want):
    Q = [A, A + 4096, A + 8192, A + 12288, A + 16384, A + 20480]
    for shared in (0, 1):
        assert lib.birkhoff_eot_fwd(Q[0], Q[1], Q[2], shared, Q[3], Q[4], Q[5], B, n, m, eta, tol, it, None) == want
        assert lib.birkhoff_eot_fwd(Q[0], Q[1], Q[2], shared, Q[3], Q[4], None, B, n, m, eta, tol, it, None) == want


def test_eot_null_and_misaligned_pointers(lib):
    """Every call here is rejected on the host (none may reach a launch: the
    addresses are fake)."""
    Q = [A, A + 4096, A + 8192, A + 12288, A + 16384]   # cost, a, b, T, dual

    def call(p, shared, iters=None):
        return lib.birkhoff_eot_fwd(p[0], p[1], p[2], shared, p[3], p[4], iters, 9, 3, 5, 0.5, 1e-6, 50, None)

    for k in range(5):
        for shared in (0, 1):
            ptrs = list(Q)
            ptrs[k] = None
            assert call(ptrs, shared) == EINVAL
            # per-problem marginals and the matrices need 16 bytes, shared marginals 4
            ptrs[k] = Q[k] + (2 if (shared and k in (1, 2)) else 4)
            assert call(ptrs, shared) == EALIGN
    assert call(Q, 0, iters=A + 24578) == EALIGN


def test_eot_backward_argument_checks(lib):
    # birkhoff_eot_bwd(T, dT, a, shared, dcost, B, n, m, eta, stream)
    Q = [A, A + 4096, A + 8192, A + 12288]
    assert lib.birkhoff_eot_bwd(Q[0], Q[1], Q[2], 0, Q[3], -1, 4, 6, 0.5, None) == EINVAL
    assert lib.birkhoff_eot_bwd(Q[0], Q[1], Q[2], 0, Q[3], 5, 4, 1, 0.5, None) == EINVAL
    assert lib.birkhoff_eot_bwd(Q[0], Q[1], Q[2], 0, Q[3], 5, 9, 6, 0.5, None) == EINVAL
    assert lib.birkhoff_eot_bwd(Q[0], Q[1], Q[2], 0, Q[3], 5, 4, 6, 0.0, None) == EINVAL
    assert lib.birkhoff_eot_bwd(Q[0], Q[1], Q[2], 0, Q[3], 5, 4, 6, math.nan, None) == EINVAL
    assert lib.birkhoff_eot_bwd(None, None, None, 0, None, 0, 4, 6, 0.5, None) == 0
    for k in range(4):
        ptrs = list(Q)
        ptrs[k] = None
        assert lib.birkhoff_eot_bwd(ptrs[0], ptrs[1], ptrs[2], 0, ptrs[3], 5, 4, 6, 0.5, None) == EINVAL
        ptrs[k] = Q[k] + 8
        assert lib.birkhoff_eot_bwd(ptrs[0], ptrs[1], ptrs[2], 0, ptrs[3], 5, 4, 6, 0.5, None) == EALIGN


# birkhoff_fwd_mix(logits, x, T, dual, y, B, n, C, tol, max_iter, stream)
@pytest.mark.parametrize("B,n,C,tol,it,want", [
    (-1, 4, 64, 1e-6, 50, EINVAL),
    (5, 8, 64, 1e-6, 50, EINVAL),
    (5, 3, 64, 1e-6, 50, EINVAL),
    (5, 4, -8, 1e-6, 50, EINVAL),
    (5, 4, 12, 1e-6, 50, "bf16"),          # a multiple of 4 but not of 8: fp32 only
    (5, 4, 6, 1e-6, 50, EINVAL),
    (5, 4, 1 << 29, 1e-6, 50, EINVAL),
    (1 << 40, 4, 1 << 20, 1e-6, 50, EINVAL),
    (5, 4, 64, 0.0, 50, EINVAL),
    (5, 4, 64, math.nan, 50, EINVAL),
    (5, 4, 64, 1e-6, 0, EINVAL),
    (0, 4, 64, 1e-6, 50, 0),
])
def test_mix_forward_argument_checks(lib, B, n, C, tol, it, want):
    Q = [A, A + 4096, A + 8192, A + 12288, A + 16384]
    if want == "bf16":
        assert lib.birkhoff_fwd_mix_bf16(*Q, B, n, C, tol, it, None) == EINVAL
        return
    assert lib.birkhoff_fwd_mix(*Q, B, n, C, tol, it, None) == want
    assert lib.birkhoff_fwd_mix_bf16(*Q, B, n, C, tol, it, None) == want


def test_mix_null_and_misaligned_pointers(lib):
    """Every call here is rejected on the host (none may reach a launch)."""
    Q = [A, A + 4096, A + 8192, A + 12288, A + 16384]   # logits, x, T, dual, y
    for k in range(5):
        ptrs = list(Q)
        ptrs[k] = None
        assert lib.birkhoff_fwd_mix(*ptrs, 9, 4, 64, 1e-6, 50, None) == EINVAL
        ptrs[k] = Q[k] + 4
        assert lib.birkhoff_fwd_mix(*ptrs, 9, 4, 64, 1e-6, 50, None) == EALIGN
        assert lib.birkhoff_fwd_mix_bf16(*ptrs, 9, 4, 64, 1e-6, 50, None) == EALIGN
    R = [A, A + 4096, A + 8192, A + 12288, A + 16384]   # T, x, dy, dx, dH
    assert lib.birkhoff_mix_bwd(*R, -1, 4, 64, None) == EINVAL
    assert lib.birkhoff_mix_bwd(*R, 5, 8, 64, None) == EINVAL
    assert lib.birkhoff_mix_bwd(*R, 5, 4, 6, None) == EINVAL
    assert lib.birkhoff_mix_bwd_bf16(*R, 5, 4, 12, None) == EINVAL
    assert lib.birkhoff_mix_bwd(None, None, None, None, None, 0, 4, 64, None) == 0
    for k in range(5):
        ptrs = list(R)
        ptrs[k] = None
        assert lib.birkhoff_mix_bwd(*ptrs, 9, 4, 64, None) == EINVAL
        ptrs[k] = R[k] + 8
        assert lib.birkhoff_mix_bwd(*ptrs, 9, 4, 64, None) == EALIGN
        assert lib.birkhoff_mix_bwd_bf16(*ptrs, 9, 4, 64, None) == EALIGN


def test_clock_probe_argument_checks(lib):
    khz = ctypes.c_int(0)
    ref = ctypes.byref(khz)
    assert lib.birkhoff_clock_probe(None, 4, 100, ref, None) == EINVAL
    assert lib.birkhoff_clock_probe(A, 4, 100, None, None) == EINVAL
    for blocks, ticks in ((0, 100), (-1, 100), (65537, 100), (4, 0), (4, -5), (4, (1 << 20) + 1)):
        assert lib.birkhoff_clock_probe(A, blocks, ticks, ref, None) == EINVAL, (blocks, ticks)
    assert lib.birkhoff_clock_probe(A + 8, 4, 100, ref, None) == EALIGN


ELAUNCH_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import birkhoff_projection_amd as bp
lib = bp.load_library()
A = 1 << 20
khz = ctypes.c_int(0)
codes = [lib.birkhoff_fwd(A, A + 4096, A + 8192, 5, 4, 1e-6, 50, None),
         lib.birkhoff_fwd_bwd(A, A + 4096, A + 8192, A + 12288, A + 16384, 5, 8, 1e-6, 50, None),
         lib.sinkhorn_fwd(A, A + 4096, 5, 4, 20, None),
         lib.birkhoff_clock_probe(A, 4, 100, ctypes.byref(khz), None)]
print(" ".join(map(str, codes)))
"""


@pytest.mark.skipif(pathlib.Path("/dev/kfd").exists(),
                    reason="needs a machine without a GPU: the valid calls here use fake addresses, "
                           "which only a launch that fails may be given")
def test_launch_failure_is_reported():
    """Calls that pass every argument check reach the launch; where the HIP
    runtime has no device to launch on, each returns BIRKHOFF_ELAUNCH (the
    launch's own status) instead of crashing or reporting success."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", ELAUNCH_SCRIPT, str(ROOT)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["-3"] * 4, r.stdout


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import birkhoff_projection_amd as mod
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "_LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(RuntimeError, match="not built"):
        mod.load_library()
