"""float64 CPU oracle for the KL Birkhoff projection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``birkhoff_projection_amd`` and its binding) never imports it, and this package
imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, OpenMP across
independent matrices); this module only compiles it with gcc and marshals
numpy arrays through ctypes.  See the header of ``oracle.c`` for the passages
of "Accelerating Birkhoff Projection for Manifold-Constrained
Hyper-Connections" that each function follows.

The Birkhoff functions take float64 arrays of shape [B, n, n] (row-major); the
eot_* functions take a cost [B, n, m] with marginals a, b and eta.  All return
float64 arrays.  Inputs stored as fp32 or bf16 are decoded exactly to float64
by the caller before they get here.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None

SK_CAP_DEFAULT = 10_000


def build(force: bool = True) -> pathlib.Path:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("ORACLE_LIB")   # a deliberately broken build, for the mutation tests
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB_PATH))
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i64, ci, cd = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_threads.restype = ci
    lib.oracle_threads.argtypes = []
    lib.oracle_nmax.restype = ci
    lib.oracle_nmax.argtypes = []
    lib.oracle_sinkhorn_tol.restype = ci
    lib.oracle_sinkhorn_tol.argtypes = [dp, i64, ci, cd, ci, dp, dp, ip, ip]
    lib.oracle_sinkhorn_k.restype = ci
    lib.oracle_sinkhorn_k.argtypes = [dp, i64, ci, ci, dp]
    lib.oracle_newton.restype = ci
    lib.oracle_newton.argtypes = [dp, i64, ci, cd, ci, dp, dp, ip]
    lib.oracle_project.restype = ci
    lib.oracle_project.argtypes = [dp, i64, ci, ci, dp, dp, ip]
    lib.oracle_bwd.restype = ci
    lib.oracle_bwd.argtypes = [dp, dp, i64, ci, dp]
    lib.oracle_eot_sinkhorn_tol.restype = ci
    lib.oracle_eot_sinkhorn_tol.argtypes = [dp, dp, dp, i64, ci, ci, cd, cd, ci, dp, dp, ip, ip]
    lib.oracle_eot_newton.restype = ci
    lib.oracle_eot_newton.argtypes = [dp, dp, dp, i64, ci, ci, cd, cd, ci, dp, dp, ip]
    lib.oracle_eot_project.restype = ci
    lib.oracle_eot_project.argtypes = [dp, dp, dp, i64, ci, ci, cd, ci, dp, dp, ip]
    lib.oracle_eot_bwd.restype = ci
    lib.oracle_eot_bwd.argtypes = [dp, dp, dp, dp, i64, ci, ci, cd, dp]
    lib.oracle_mix.restype = ci
    lib.oracle_mix.argtypes = [dp, dp, i64, ci, i64, dp]
    lib.oracle_mix_bwd.restype = ci
    lib.oracle_mix_bwd.argtypes = [dp, dp, dp, i64, ci, i64, dp, dp]
    _lib = lib
    return lib


def _mat(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.ndim == 2:
        a = a[None]
    if a.ndim != 3 or a.shape[1] != a.shape[2]:
        raise ValueError("expected [B, n, n] or [n, n], got %r" % (a.shape,))
    return a


def _p(a: np.ndarray, ct=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _check(rc: int, what: str) -> None:
    if rc < 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().oracle_threads())


def project(H, sk_cap: int = SK_CAP_DEFAULT):
    """Reference projection T = proj_KL(exp(H)) onto B_n.

    Returns (T [B,n,n], beta [B,n] with beta_n = 0, status [B] int32), where
    status 0 = Sinkhorn converged to 1e-13 and agrees with Newton to 1e-12,
    1 = Sinkhorn capped but Newton converged and passed the fixed-point check,
    negative = not certified.
    """
    H = _mat(H)
    B, n, _ = H.shape
    T = np.empty_like(H)
    beta = np.empty((B, n))
    st = np.empty(B, dtype=np.int32)
    _check(_load().oracle_project(_p(H), B, n, int(sk_cap), _p(T), _p(beta), _p(st, ctypes.c_int32)),
           "project")
    return T, beta, st


def sinkhorn_tol(H, tol: float = 1e-13, cap: int = SK_CAP_DEFAULT):
    """Sinkhorn-Knopp to marginal residual <= tol. Returns (T, beta, sweeps, converged)."""
    H = _mat(H)
    B, n, _ = H.shape
    T = np.empty_like(H)
    beta = np.empty((B, n))
    sw = np.empty(B, dtype=np.int32)
    cv = np.empty(B, dtype=np.int32)
    _check(_load().oracle_sinkhorn_tol(_p(H), B, n, float(tol), int(cap), _p(T), _p(beta),
                                       _p(sw, ctypes.c_int32), _p(cv, ctypes.c_int32)),
           "sinkhorn_tol")
    return T, beta, sw, cv.astype(bool)


def sinkhorn_k(H, K: int = 20):
    """Exactly K Sinkhorn-Knopp sweeps from v = 1 (the fixed-iteration baseline)."""
    H = _mat(H)
    B, n, _ = H.shape
    T = np.empty_like(H)
    _check(_load().oracle_sinkhorn_k(_p(H), B, n, int(K), _p(T)), "sinkhorn_k")
    return T


def newton(H, tol: float = 1e-13, max_iter: int = 500):
    """float64 Newton on the reduced dual. Returns (T, beta, iters); iters -1 = tol not met."""
    H = _mat(H)
    B, n, _ = H.shape
    T = np.empty_like(H)
    beta = np.empty((B, n))
    it = np.empty(B, dtype=np.int32)
    _check(_load().oracle_newton(_p(H), B, n, float(tol), int(max_iter), _p(T), _p(beta),
                                 _p(it, ctypes.c_int32)), "newton")
    return T, beta, it


def bwd(T, G):
    """eq (13) backward at projected matrices T with upstream G; returns dH = d<G,T>/dH."""
    T = _mat(T)
    G = _mat(G)
    if G.shape != T.shape:
        raise ValueError("T and G shapes differ")
    B, n, _ = T.shape
    dH = np.empty_like(T)
    rc = _load().oracle_bwd(_p(T), _p(G), B, n, _p(dH))
    _check(rc, "bwd")
    return dH


# ---------------------------------------------------------------------------
# General small entropic OT: cost M [B, n, m], marginals a [B, n], b [B, m]
# (or [n], [m], shared by every problem), regularisation eta > 0.
# ---------------------------------------------------------------------------

def _eot_args(M, a, b):
    M = np.ascontiguousarray(np.asarray(M, dtype=np.float64))
    if M.ndim == 2:
        M = M[None]
    if M.ndim != 3:
        raise ValueError("expected a cost of shape [B, n, m] or [n, m], got %r" % (M.shape,))
    B, n, m = M.shape
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    a = np.ascontiguousarray(np.broadcast_to(a, (B, n)))
    b = np.ascontiguousarray(np.broadcast_to(b, (B, m)))
    return M, a, b, B, n, m


def eot_project(M, a, b, eta: float = 1.0, sk_cap: int = SK_CAP_DEFAULT):
    """Reference plan of min <T, M> - eta h(T) over T with T 1 = a, T^T 1 = b.

    Returns (T [B,n,m], beta [B,m] with beta_m = 0, status [B]); status as in
    project()."""
    M, a, b, B, n, m = _eot_args(M, a, b)
    T = np.empty_like(M)
    beta = np.empty((B, m))
    st = np.empty(B, dtype=np.int32)
    _check(_load().oracle_eot_project(_p(M), _p(a), _p(b), B, n, m, float(eta), int(sk_cap), _p(T), _p(beta),
                                      _p(st, ctypes.c_int32)), "eot_project")
    return T, beta, st


def eot_sinkhorn_tol(M, a, b, eta: float = 1.0, tol: float = 1e-13, cap: int = SK_CAP_DEFAULT):
    """Sinkhorn-Knopp (eq 7) to marginal residual <= tol. Returns (T, beta, sweeps, converged)."""
    M, a, b, B, n, m = _eot_args(M, a, b)
    T = np.empty_like(M)
    beta = np.empty((B, m))
    sw = np.empty(B, dtype=np.int32)
    cv = np.empty(B, dtype=np.int32)
    _check(_load().oracle_eot_sinkhorn_tol(_p(M), _p(a), _p(b), B, n, m, float(eta), float(tol), int(cap), _p(T),
                                           _p(beta), _p(sw, ctypes.c_int32), _p(cv, ctypes.c_int32)),
           "eot_sinkhorn_tol")
    return T, beta, sw, cv.astype(bool)


def eot_newton(M, a, b, eta: float = 1.0, tol: float = 1e-13, max_iter: int = 500):
    """float64 Newton on the reduced dual of eq (8). Returns (T, beta, iters); iters -1 = tol not met."""
    M, a, b, B, n, m = _eot_args(M, a, b)
    T = np.empty_like(M)
    beta = np.empty((B, m))
    it = np.empty(B, dtype=np.int32)
    _check(_load().oracle_eot_newton(_p(M), _p(a), _p(b), B, n, m, float(eta), float(tol), int(max_iter), _p(T),
                                     _p(beta), _p(it, ctypes.c_int32)), "eot_newton")
    return T, beta, it


def eot_bwd(T, G, a, b, eta: float = 1.0):
    """eq (13): D = d<G, T*>/dM at plans T with upstream G."""
    T, a, b, B, n, m = _eot_args(T, a, b)
    G = np.ascontiguousarray(np.asarray(G, dtype=np.float64)).reshape(T.shape)
    D = np.empty_like(T)
    _check(_load().oracle_eot_bwd(_p(T), _p(G), _p(a), _p(b), B, n, m, float(eta), _p(D)), "eot_bwd")
    return D


# ---------------------------------------------------------------------------
# mHC consumer: y = T x for the n x C hidden matrix x of each token.
# ---------------------------------------------------------------------------

def _streams(x, B, n):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if x.ndim != 3 or x.shape[0] != B or x.shape[1] != n:
        raise ValueError("expected [%d, %d, C], got %r" % (B, n, x.shape))
    return x


def mix(T, x):
    """y = T x per token: T [B, n, n], x [B, n, C] -> y [B, n, C]."""
    T = _mat(T)
    B, n, _ = T.shape
    x = _streams(x, B, n)
    y = np.empty_like(x)
    _check(_load().oracle_mix(_p(T), _p(x), B, n, x.shape[2], _p(y)), "mix")
    return y


def mix_bwd(T, x, dy):
    """Backward of y = T x: returns (dx = T^T dy, dT = dy x^T)."""
    T = _mat(T)
    B, n, _ = T.shape
    x = _streams(x, B, n)
    dy = _streams(dy, B, n)
    if dy.shape != x.shape:
        raise ValueError("x and dy shapes differ")
    dx = np.empty_like(x)
    dT = np.empty_like(T)
    _check(_load().oracle_mix_bwd(_p(T), _p(x), _p(dy), B, n, x.shape[2], _p(dx), _p(dT)), "mix_bwd")
    return dx, dT
