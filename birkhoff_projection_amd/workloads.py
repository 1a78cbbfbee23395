"""Seeded synthetic workloads for the Birkhoff projection.

This module holds random inputs and storage encodings only -- none of the
projection's arithmetic -- so that the HIP path and the float64 oracle can be
fed the very same numbers.  It imports nothing else from the package.

Recipe (every workload): a ``numpy.random.Generator(PCG64(seed))`` draws float64
standard normals, which are scaled, then rounded to fp32 (round-to-nearest-
even) and, for bf16 storage, rounded again fp32 -> bf16 (RNE).  Logits use
``seed``; the upstream gradient dL/dT uses ``seed + 100``.  Matrices are
row-major and stored back to back, shape [B, n, n].

The distributions follow the pages' experiments ("Accelerating Birkhoff
Projection for Manifold-Constrained Hyper-Connections", section 5: N(0,1),
N(0,10^2)) and the benchmark shapes below; no dataset is involved.

General entropic OT workloads (EOT_WORKLOADS, the problem of section 2.3 with
a cost, marginals and eta): costs are drawn like logits (seed), the upstream
dL/dT from seed + 100, and the marginals from seed + 200 as dyadic
rationals k / 2^20 (k integers summing to 2^20), so that a and b are exact in
fp32, sum to exactly 1 in any precision, and the problem has an exact
solution whether it is read in fp32 or float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

_CHUNK = 1 << 20  # matrices drawn per generator call (bounds host memory)


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    B: int
    n: int
    io: str                      # storage of logits / T / dT / dH: "f32" or "bf16"
    logits: Tuple                # recipe, see make_logits
    upstream: Optional[Tuple]    # recipe for dL/dT, None if forward only
    passes: str                  # "fwd+bwd" or "fwd"
    seed: int
    tol: float = 1e-6
    max_iter: int = 50
    sk_cap: int = 10_000         # oracle Sinkhorn cap for the reference
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "pr1": Workload(
        key="pr1", title="4x4 fp32, B=4096, H~N(0,1), dT~N(0,1)",
        B=4096, n=4, io="f32", logits=("normal", 1.0), upstream=("normal", 1.0),
        passes="fwd+bwd", seed=1),
    "hard": Workload(
        key="hard", title="4x4 fp32, B=1,048,576, H~N(0,s^2), s per matrix from {1,3,5,8}",
        B=1 << 20, n=4, io="f32", logits=("sigma_mix", (1.0, 3.0, 5.0, 8.0)), upstream=None,
        passes="fwd", seed=2, max_iter=100, sk_cap=5_000),
    "train": Workload(
        key="train", title="4x4 fp32, B=16x4096x32=2,097,152, H~N(0,0.5^2)+2I, dT~N(0,0.1^2)",
        B=16 * 4096 * 32, n=4, io="f32", logits=("near_identity", 0.5, 2.0),
        upstream=("normal", 0.1), passes="fwd+bwd", seed=3),
    "n8": Workload(
        key="n8", title="8x8 fp32, B=1,048,576, H~N(0,1), dT~N(0,1)",
        B=1 << 20, n=8, io="f32", logits=("normal", 1.0), upstream=("normal", 1.0),
        passes="fwd+bwd", seed=4),
    "bw": Workload(
        key="bw", title="4x4 bf16 storage, B=16,777,216, H~N(0,1), dT~N(0,1)",
        B=1 << 24, n=4, io="bf16", logits=("normal", 1.0), upstream=("normal", 1.0),
        passes="fwd+bwd", seed=5),
}


# The timing shape of the pages' Table 3 (section 5): 4x4 logits ~ N(0, 10^2) at
# five batch sizes, forward and forward + backward.  A context report, not a
# benchmark line: one workload per batch size, all from seed 8.
PAGES_SHAPE_BATCHES = (512, 2048, 8192, 32768, 131072)


def pages_shape_workload(B: int) -> Workload:
    return Workload(key="shape%d" % B, title="4x4 fp32, B=%d, H~N(0,10^2), dT~N(0,1)" % B, B=B, n=4, io="f32",
                    logits=("normal", 10.0), upstream=("normal", 1.0), passes="fwd+bwd", seed=8, max_iter=100,
                    sk_cap=5_000)

def _draw(recipe: Tuple, B: int, n: int, seed: int, m: Optional[int] = None) -> np.ndarray:
    """fp32 [B, n, m] (m defaults to n) values for a recipe (scaling done in float64, then rounded)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kind = recipe[0]
    m = n if m is None else int(m)
    out = np.empty((B, n, m), dtype=np.float32)
    if kind == "normal":
        sigma = float(recipe[1])
        for s in range(0, B, _CHUNK):
            e = min(B, s + _CHUNK)
            out[s:e] = sigma * rng.standard_normal((e - s, n, m))
    elif kind == "sigma_mix":
        sigmas = np.asarray(recipe[1], dtype=np.float64)
        idx = rng.integers(0, len(sigmas), size=B)          # sigma index first
        for s in range(0, B, _CHUNK):
            e = min(B, s + _CHUNK)
            z = rng.standard_normal((e - s, n, m))
            out[s:e] = sigmas[idx[s:e]][:, None, None] * z
    elif kind == "near_identity":
        sigma, diag = float(recipe[1]), float(recipe[2])
        eye = np.eye(n, m) * diag
        for s in range(0, B, _CHUNK):
            e = min(B, s + _CHUNK)
            out[s:e] = sigma * rng.standard_normal((e - s, n, m)) + eye
    else:
        raise ValueError("unknown recipe %r" % (kind,))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_logits(w: Workload, B: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    """Logits H~ for workload w: fp32 [B, n, n], or uint16 bf16 bits when w.io == 'bf16'."""
    B = w.B if B is None else int(B)
    x = _draw(w.logits, B, w.n, w.seed if seed is None else seed)
    return f32_to_bf16_bits(x) if w.io == "bf16" else x


def make_upstream(w: Workload, B: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    """Upstream gradient dL/dT for workload w (same storage rule as the logits)."""
    if w.upstream is None:
        raise ValueError("workload %s is forward only" % w.key)
    B = w.B if B is None else int(B)
    x = _draw(w.upstream, B, w.n, (w.seed + 100) if seed is None else seed)
    return f32_to_bf16_bits(x) if w.io == "bf16" else x


def decode_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 view of stored inputs/outputs (fp32 array or bf16 bit patterns)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def bytes_per_projection(n: int, io: str, passes: str) -> int:
    """Algorithmic HBM bytes per projection: each input read once, each output written once.

    fwd: logits + T (n*n elements of the storage type each) + dual (n fp32);
    bwd: logits + dual + dT + dH;
    fused (forward and backward in one launch): logits + dT + T + dual + dH;
    fwd+bwd: the two separate passes.
    """
    s = 2 if io == "bf16" else 4
    fwd = 2 * n * n * s + 4 * n
    bwd = 3 * n * n * s + 4 * n
    if passes == "fwd":
        return fwd
    if passes == "bwd":
        return bwd
    if passes == "fused":
        return 4 * n * n * s + 4 * n
    if passes == "fwd+bwd":
        return fwd + bwd
    raise ValueError("unknown passes %r" % (passes,))


# ---------------------------------------------------------------------------
# General small entropic OT (cost M, marginals a and b, eta)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class EotWorkload:
    key: str
    title: str
    B: int
    n: int
    m: int
    eta: float                   # exactly representable in fp32
    cost: Tuple                  # recipe for M, as for logits
    marginals: Tuple             # ("dyadic", lo, hi): weights ~ U(lo, hi), see make_marginals
    upstream: Tuple              # recipe for dL/dT
    seed: int
    shared: bool = False         # one (a, b) pair for the whole batch
    tol: float = 1e-6
    max_iter: int = 50
    sk_cap: int = 10_000


EOT_WORKLOADS = {
    "eot": EotWorkload(
        key="eot", title="4x6 fp32 entropic OT, B=1,048,576, M~N(0,1), eta=1/2, per-problem marginals "
                         "~U(0.5,1.5) normalised, dT~N(0,1)",
        B=1 << 20, n=4, m=6, eta=0.5, cost=("normal", 1.0), marginals=("dyadic", 0.5, 1.5),
        upstream=("normal", 1.0), seed=6),
}


def make_marginals(recipe: Tuple, B: int, k: int, seed: int) -> np.ndarray:
    """fp32 [B, k] marginals: weights w ~ U(lo, hi) in float64, turned into integers
    q = floor(w / sum(w) * 2^20) whose shortfall from 2^20 is added to the largest,
    then a = q / 2^20 (exact in fp32; every row sums to exactly 1)."""
    kind, lo, hi = recipe
    if kind != "dyadic":
        raise ValueError("unknown marginal recipe %r" % (kind,))
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.uniform(lo, hi, size=(B, k))
    q = np.floor(w / w.sum(1, keepdims=True) * (1 << 20)).astype(np.int64)
    q[np.arange(B), q.argmax(1)] += (1 << 20) - q.sum(1)
    return (q / float(1 << 20)).astype(np.float32)


def make_eot(w: EotWorkload, B: Optional[int] = None, seed: Optional[int] = None):
    """(cost [B, n, m], a, b) fp32 for workload w; a, b are [B, n], [B, m], or [n], [m] when shared."""
    B = w.B if B is None else int(B)
    sd = w.seed if seed is None else seed
    M = _draw(w.cost, B, w.n, sd, w.m)
    nb = 1 if w.shared else B
    a = make_marginals(w.marginals, nb, w.n, sd + 200)
    b = make_marginals(w.marginals, nb, w.m, sd + 300)
    return (M, a[0], b[0]) if w.shared else (M, a, b)


def make_eot_upstream(w: EotWorkload, B: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    B = w.B if B is None else int(B)
    return _draw(w.upstream, B, w.n, (w.seed + 100) if seed is None else seed, w.m)


def eot_bytes_per_problem(n: int, m: int, passes: str, shared: bool) -> int:
    """Algorithmic HBM bytes per problem (fp32), each input read once, each output written once.

    fwd: cost + T (n*m each) + dual (m) + the marginals (n + m) unless shared;
    bwd: T + dT + dcost (n*m each) + a (n) unless shared."""
    fwd = 4 * (2 * n * m + m + (0 if shared else n + m))
    bwd = 4 * (3 * n * m + (0 if shared else n))
    if passes == "fwd":
        return fwd
    if passes == "bwd":
        return bwd
    if passes == "fwd+bwd":
        return fwd + bwd
    raise ValueError("unknown passes %r" % (passes,))


# ---------------------------------------------------------------------------
# The projection's consumer: y = H_res x for per-token hidden states x [B, 4, C]
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MixWorkload:
    key: str
    title: str
    B: int                       # tokens (one 4 x 4 logit matrix each)
    C: int                       # features per stream
    io: str                      # storage of x, y, dy, dx: "f32" or "bf16"
    logits: Tuple                # recipe for the 4 x 4 logits (fp32)
    hidden: Tuple                # recipe for x
    upstream: Tuple              # recipe for dL/dy
    seed: int
    tol: float = 1e-6
    max_iter: int = 50


MIX_WORKLOADS = {
    "mix": MixWorkload(
        key="mix", title="4x4 projection + y = T x, B=16x4096=65,536 tokens, C=4096 bf16 streams, "
                         "H~N(0,0.5^2)+2I, x~N(0,1), dy~N(0,1)",
        B=16 * 4096, C=4096, io="bf16", logits=("near_identity", 0.5, 2.0), hidden=("normal", 1.0),
        upstream=("normal", 1.0), seed=7),
}


def _draw_streams(recipe: Tuple, B: int, C: int, seed: int, io: str) -> np.ndarray:
    """[B, 4, C] hidden states (fp32, or bf16 bit patterns), drawn 2^22 values at a time."""
    kind, sigma = recipe
    if kind != "normal":
        raise ValueError("unknown stream recipe %r" % (kind,))
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((B, 4, C), dtype=np.uint16 if io == "bf16" else np.float32)
    flat = out.reshape(-1)
    step = 1 << 22
    for s in range(0, flat.size, step):
        e = min(flat.size, s + step)
        v = (float(sigma) * rng.standard_normal(e - s)).astype(np.float32)
        flat[s:e] = f32_to_bf16_bits(v) if io == "bf16" else v
    return out


def make_mix(w: MixWorkload, B: Optional[int] = None, C: Optional[int] = None, seed: Optional[int] = None):
    """(logits [B, 4, 4] fp32, x [B, 4, C], dy [B, 4, C]) for workload w; logits use seed,
    x seed + 400, dy seed + 500."""
    B = w.B if B is None else int(B)
    C = w.C if C is None else int(C)
    sd = w.seed if seed is None else seed
    H = _draw(w.logits, B, 4, sd)
    x = _draw_streams(w.hidden, B, C, sd + 400, w.io)
    dy = _draw_streams(w.upstream, B, C, sd + 500, w.io)
    return H, x, dy


def mix_bytes_per_token(C: int, io: str, passes: str) -> int:
    """Algorithmic HBM bytes per token, each input read once, each output written once.

    fwd (birkhoff_fwd_mix): logits + T (16 fp32 each) + dual (4 fp32) + x + y (4C elements each);
    bwd (birkhoff_mix_bwd): T + dH (16 fp32 each) + x + dy + dx (4C elements each)."""
    s = 2 if io == "bf16" else 4
    fwd = 4 * (16 + 16 + 4) + 2 * 4 * C * s
    bwd = 4 * (16 + 16) + 3 * 4 * C * s
    if passes == "fwd":
        return fwd
    if passes == "bwd":
        return bwd
    if passes == "fwd+bwd":
        return fwd + bwd
    raise ValueError("unknown passes %r" % (passes,))
