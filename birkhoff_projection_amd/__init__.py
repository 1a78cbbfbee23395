"""MI355X-native batched KL projection onto the Birkhoff polytope (mHC).

Thin Python binding over libbirkhoff.so (C ABI in include/birkhoff.h).  The
functions below carry the ABI's names and only marshal arguments: they check
shapes, dtypes, devices and contiguity of torch tensors, pass raw device
pointers and torch's current HIP stream, and turn error codes into
exceptions.  Every step of the computation runs in the HIP kernels; there is
no CPU or PyTorch fallback.  If the library is not built, every call raises.

    import torch, birkhoff_projection_amd as bp
    H = torch.randn(4096, 4, 4, device="cuda")
    T, dual = bp.project(H)                      # forward, allocating outputs
    T = bp.BirkhoffProjection.apply(H)           # autograd: backward by eq (13)
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Optional

__all__ = [
    "BirkhoffError", "library_path", "load_library",
    "birkhoff_fwd", "birkhoff_fwd_ex", "birkhoff_bwd", "birkhoff_bwd_from_T", "sinkhorn_fwd",
    "birkhoff_fwd_bf16", "birkhoff_bwd_bf16", "birkhoff_fwd_bwd", "birkhoff_fwd_bwd_bf16",
    "birkhoff_eot_fwd", "birkhoff_eot_bwd",
    "birkhoff_fwd_mix", "birkhoff_fwd_mix_bf16", "birkhoff_mix_bwd", "birkhoff_mix_bwd_bf16",
    "birkhoff_strerror", "birkhoff_abi_version", "ClockProbe",
    "project", "project_bwd", "project_fwd_bwd", "sinkhorn", "BirkhoffProjection",
    "eot_plan", "eot_plan_bwd", "EntropicOT",
    "project_mix", "project_mix_bwd", "ProjectMix",
]

_PKG = pathlib.Path(__file__).resolve().parent
_LIB_PATH = _PKG / "libbirkhoff.so"
_lib = None


class BirkhoffError(RuntimeError):
    """A libbirkhoff call returned a non-zero code."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s (code %d)" % (where, birkhoff_strerror(code), code))


def library_path() -> pathlib.Path:
    return _LIB_PATH


def load_library():
    """Load libbirkhoff.so (built in-tree by birkhoff_projection_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError("libbirkhoff.so is not built (%s); run `python -m birkhoff_projection_amd.build` "
                           "or __graft_entry__.build()" % _LIB_PATH)
    lib = ctypes.CDLL(str(_LIB_PATH))
    vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sig = {
        "birkhoff_fwd": [vp, vp, vp, i64, ci, cf, ci, vp],
        "birkhoff_fwd_ex": [vp, vp, vp, vp, vp, i64, ci, cf, ci, vp],
        "birkhoff_bwd": [vp, vp, vp, vp, i64, ci, vp],
        "birkhoff_bwd_from_T": [vp, vp, vp, i64, ci, vp],
        "sinkhorn_fwd": [vp, vp, i64, ci, ci, vp],
        "birkhoff_fwd_bf16": [vp, vp, vp, i64, ci, cf, ci, vp],
        "birkhoff_bwd_bf16": [vp, vp, vp, vp, i64, ci, vp],
        "birkhoff_fwd_bwd": [vp, vp, vp, vp, vp, i64, ci, cf, ci, vp],
        "birkhoff_fwd_bwd_bf16": [vp, vp, vp, vp, vp, i64, ci, cf, ci, vp],
        "birkhoff_eot_fwd": [vp, vp, vp, ci, vp, vp, vp, i64, ci, ci, cf, cf, ci, vp],
        "birkhoff_eot_bwd": [vp, vp, vp, ci, vp, i64, ci, ci, cf, vp],
        "birkhoff_fwd_mix": [vp, vp, vp, vp, vp, i64, ci, i64, cf, ci, vp],
        "birkhoff_fwd_mix_bf16": [vp, vp, vp, vp, vp, i64, ci, i64, cf, ci, vp],
        "birkhoff_mix_bwd": [vp, vp, vp, vp, vp, i64, ci, i64, vp],
        "birkhoff_mix_bwd_bf16": [vp, vp, vp, vp, vp, i64, ci, i64, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ci
    lib.birkhoff_clock_probe.argtypes = [vp, ci, ci, ctypes.POINTER(ci), vp]
    lib.birkhoff_clock_probe.restype = ci
    lib.birkhoff_strerror.argtypes = [ci]
    lib.birkhoff_strerror.restype = ctypes.c_char_p
    lib.birkhoff_abi_version.argtypes = []
    lib.birkhoff_abi_version.restype = ci
    _lib = lib
    return lib


def birkhoff_strerror(code: int) -> str:
    return load_library().birkhoff_strerror(int(code)).decode()


def birkhoff_abi_version() -> int:
    return int(load_library().birkhoff_abi_version())


# ---------------------------------------------------------------- marshalling

_torch_mod = None


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch
        _torch_mod = torch
    return _torch_mod


def _stream_handle(stream, device):
    if stream is None:
        stream = _torch().cuda.current_stream(device)
    return stream.cuda_stream


def _mats(x, name, dtype, B=None, n=None):
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == dtype and x.is_contiguous():
        shp = x.shape   # the common case in one pass; the checks below name what is wrong
        if len(shp) == 3 and shp[1] == shp[2] and (B is None or (shp[0] == B and shp[1] == n)):
            return x
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not x.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if x.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, x.dtype))
    if x.dim() != 3 or x.shape[1] != x.shape[2]:
        raise ValueError("%s must have shape [B, n, n], got %s" % (name, tuple(x.shape)))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if B is not None and (x.shape[0] != B or x.shape[1] != n):
        raise ValueError("%s must have shape [%d, %d, %d], got %s" % (name, B, n, n, tuple(x.shape)))
    return x


def _vec(x, name, B, n, dtype):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != dtype or not x.is_contiguous():
        raise ValueError("%s must be a contiguous %s GPU tensor" % (name, dtype))
    if tuple(x.shape) != ((B, n) if n is not None else (B,)):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), (B, n) if n else (B,)))
    return x


def _same_device(*ts):
    i = ts[0].get_device()
    for t in ts[1:]:
        if t.get_device() != i:
            raise ValueError("all tensors must be on the same device")
    return ts[0].device


def _call(name, device, *args):
    """Calls the entry point with `device` current (HIP launches on the current
    device's view of the stream); the device switch is skipped when it already is."""
    torch = _torch()
    fn = getattr(_lib if _lib is not None else load_library(), name)
    if device.index == torch.cuda.current_device():
        rc = fn(*args)
    else:
        with torch.cuda.device(device):
            rc = fn(*args)
    if rc != 0:
        raise BirkhoffError(rc, name)


def _p(t):
    return t.data_ptr()   # a plain address; the entry points' argtypes make it a void*


# ------------------------------------------------------------- ABI wrappers

def birkhoff_fwd(logits, T, dual, tol: float = 1e-6, max_iter: int = 50, stream=None) -> None:
    """Forward projection into preallocated T [B,n,n] and dual [B,n] (fp32)."""
    torch = _torch()
    _mats(logits, "logits", torch.float32)
    B, n = logits.shape[0], logits.shape[1]
    _mats(T, "T", torch.float32, B, n)
    _vec(dual, "dual", B, n, torch.float32)
    dev = _same_device(logits, T, dual)
    _call("birkhoff_fwd", dev, _p(logits), _p(T), _p(dual), B, n, float(tol), int(max_iter),
          _stream_handle(stream, dev))


def birkhoff_fwd_ex(logits, T, dual, iters, tol: float = 1e-6, max_iter: int = 50, stream=None,
                    fallbacks=None) -> None:
    """As birkhoff_fwd, also writing iters [B] int32 (updates used, -1 if tol not reached)
    and, if given, fallbacks [B] int32 (how many of the updates were fallback sweeps)."""
    torch = _torch()
    _mats(logits, "logits", torch.float32)
    B, n = logits.shape[0], logits.shape[1]
    _mats(T, "T", torch.float32, B, n)
    _vec(dual, "dual", B, n, torch.float32)
    _vec(iters, "iters", B, None, torch.int32)
    if fallbacks is not None:
        _vec(fallbacks, "fallbacks", B, None, torch.int32)
        dev = _same_device(logits, T, dual, iters, fallbacks)
    else:
        dev = _same_device(logits, T, dual, iters)
    _call("birkhoff_fwd_ex", dev, _p(logits), _p(T), _p(dual), _p(iters),
          None if fallbacks is None else _p(fallbacks), B, n, float(tol), int(max_iter),
          _stream_handle(stream, dev))


def birkhoff_bwd(logits, dual, dT, dH, stream=None) -> None:
    """Backward: dH = dL/dlogits from dT = dL/dT, at the forward's dual (fp32)."""
    torch = _torch()
    _mats(logits, "logits", torch.float32)
    B, n = logits.shape[0], logits.shape[1]
    _vec(dual, "dual", B, n, torch.float32)
    _mats(dT, "dT", torch.float32, B, n)
    _mats(dH, "dH", torch.float32, B, n)
    dev = _same_device(logits, dual, dT, dH)
    _call("birkhoff_bwd", dev, _p(logits), _p(dual), _p(dT), _p(dH), B, n, _stream_handle(stream, dev))


def birkhoff_bwd_from_T(T, dT, dH, stream=None) -> None:
    """Backward from the projection T itself: dH = dL/dlogits from dT (fp32)."""
    torch = _torch()
    _mats(T, "T", torch.float32)
    B, n = T.shape[0], T.shape[1]
    _mats(dT, "dT", torch.float32, B, n)
    _mats(dH, "dH", torch.float32, B, n)
    dev = _same_device(T, dT, dH)
    _call("birkhoff_bwd_from_T", dev, _p(T), _p(dT), _p(dH), B, n, _stream_handle(stream, dev))


class ClockProbe:
    """The engine clock that kernels run at (birkhoff_clock_probe): `launch`
    enqueues the probe on a stream; `mhz` reads its result once the stream has
    passed it (it synchronises)."""

    def __init__(self, device, blocks: int = 256, ticks: int = 2000):
        torch = _torch()
        self.device = torch.device(device)
        self.blocks, self.ticks = int(blocks), int(ticks)
        self.counts = torch.zeros(2 * self.blocks, dtype=torch.int64, device=self.device)
        self.wall_khz = None

    def launch(self, stream=None) -> None:
        khz = ctypes.c_int(0)
        _call("birkhoff_clock_probe", self.device, _p(self.counts), self.blocks, self.ticks, ctypes.byref(khz),
              _stream_handle(stream, self.device))
        self.wall_khz = khz.value

    def mhz(self) -> float:
        if self.wall_khz is None:
            raise RuntimeError("ClockProbe.mhz() before launch()")
        c = self.counts.view(-1, 2).cpu().double()
        return float(c[:, 0].sum() / c[:, 1].sum()) * self.wall_khz / 1e3


def sinkhorn_fwd(logits, T, iters: int = 20, stream=None) -> None:
    """Baseline: exactly `iters` Sinkhorn-Knopp sweeps (fp32) into preallocated T."""
    torch = _torch()
    _mats(logits, "logits", torch.float32)
    B, n = logits.shape[0], logits.shape[1]
    _mats(T, "T", torch.float32, B, n)
    dev = _same_device(logits, T)
    _call("sinkhorn_fwd", dev, _p(logits), _p(T), B, n, int(iters), _stream_handle(stream, dev))


def _bf16_mats(x, name, B=None, n=None):
    """bf16 storage is passed as torch.bfloat16 (or int16 / uint16 bit patterns)."""
    torch = _torch()
    if x.dtype not in (torch.bfloat16, torch.int16, getattr(torch, "uint16", torch.int16)):
        raise TypeError("%s must be bfloat16 (or 16-bit bf16 bit patterns), got %s" % (name, x.dtype))
    return _mats(x, name, x.dtype, B, n)


def birkhoff_fwd_bf16(logits, T, dual, tol: float = 1e-6, max_iter: int = 50, stream=None) -> None:
    """Forward with bf16 storage of logits and T (fp32 arithmetic and fp32 dual)."""
    torch = _torch()
    _bf16_mats(logits, "logits")
    B, n = logits.shape[0], logits.shape[1]
    _bf16_mats(T, "T", B, n)
    _vec(dual, "dual", B, n, torch.float32)
    dev = _same_device(logits, T, dual)
    _call("birkhoff_fwd_bf16", dev, _p(logits), _p(T), _p(dual), B, n, float(tol), int(max_iter),
          _stream_handle(stream, dev))


def birkhoff_bwd_bf16(logits, dual, dT, dH, stream=None) -> None:
    """Backward with bf16 storage of logits, dT and dH (fp32 arithmetic and fp32 dual)."""
    torch = _torch()
    _bf16_mats(logits, "logits")
    B, n = logits.shape[0], logits.shape[1]
    _vec(dual, "dual", B, n, torch.float32)
    _bf16_mats(dT, "dT", B, n)
    _bf16_mats(dH, "dH", B, n)
    dev = _same_device(logits, dual, dT, dH)
    _call("birkhoff_bwd_bf16", dev, _p(logits), _p(dual), _p(dT), _p(dH), B, n, _stream_handle(stream, dev))


def birkhoff_fwd_bwd(logits, dT, T, dual, dH, tol: float = 1e-6, max_iter: int = 50, stream=None) -> None:
    """Forward and backward in one launch (fp32): T, dual as birkhoff_fwd; dH = dL/dlogits for dT."""
    torch = _torch()
    _mats(logits, "logits", torch.float32)
    B, n = logits.shape[0], logits.shape[1]
    _mats(dT, "dT", torch.float32, B, n)
    _mats(T, "T", torch.float32, B, n)
    _vec(dual, "dual", B, n, torch.float32)
    _mats(dH, "dH", torch.float32, B, n)
    dev = _same_device(logits, dT, T, dual, dH)
    _call("birkhoff_fwd_bwd", dev, _p(logits), _p(dT), _p(T), _p(dual), _p(dH), B, n, float(tol), int(max_iter),
          _stream_handle(stream, dev))


def birkhoff_fwd_bwd_bf16(logits, dT, T, dual, dH, tol: float = 1e-6, max_iter: int = 50, stream=None) -> None:
    """Forward and backward in one launch with bf16 storage (fp32 arithmetic and fp32 dual)."""
    torch = _torch()
    _bf16_mats(logits, "logits")
    B, n = logits.shape[0], logits.shape[1]
    _bf16_mats(dT, "dT", B, n)
    _bf16_mats(T, "T", B, n)
    _vec(dual, "dual", B, n, torch.float32)
    _bf16_mats(dH, "dH", B, n)
    dev = _same_device(logits, dT, T, dual, dH)
    _call("birkhoff_fwd_bwd_bf16", dev, _p(logits), _p(dT), _p(T), _p(dual), _p(dH), B, n, float(tol),
          int(max_iter), _stream_handle(stream, dev))


def _plans(x, name, B=None, n=None, m=None):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("%s must be a contiguous float32 GPU tensor" % name)
    if x.dim() != 3:
        raise ValueError("%s must have shape [B, n, m], got %s" % (name, tuple(x.shape)))
    if B is not None and tuple(x.shape) != (B, n, m):
        raise ValueError("%s must have shape %s, got %s" % (name, (B, n, m), tuple(x.shape)))
    return x


def _marginal(x, name, B, k):
    """A marginal is [B, k] (one per problem) or [k] (shared); returns the shared flag."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("%s must be a contiguous float32 GPU tensor" % name)
    if tuple(x.shape) == (k,):
        return 1
    if tuple(x.shape) == (B, k):
        return 0
    raise ValueError("%s must have shape [%d] or [%d, %d], got %s" % (name, k, B, k, tuple(x.shape)))


def birkhoff_eot_fwd(cost, a, b, T, dual, iters=None, eta: float = 1.0, tol: float = 1e-6, max_iter: int = 50,
                     stream=None) -> None:
    """General entropic OT plan: cost [B,n,m], marginals a ([B,n] or [n]) and b ([B,m] or [m]);
    writes T [B,n,m], dual [B,m] and optionally iters [B] int32."""
    torch = _torch()
    _plans(cost, "cost")
    B, n, m = cost.shape
    sa, sb = _marginal(a, "a", B, n), _marginal(b, "b", B, m)
    if sa != sb:
        raise ValueError("a and b must both be shared or both be per problem")
    _plans(T, "T", B, n, m)
    _vec(dual, "dual", B, m, torch.float32)
    ts = [cost, a, b, T, dual]
    if iters is not None:
        _vec(iters, "iters", B, None, torch.int32)
        ts.append(iters)
    dev = _same_device(*ts)
    _call("birkhoff_eot_fwd", dev, _p(cost), _p(a), _p(b), sa, _p(T), _p(dual),
          _p(iters) if iters is not None else None, B, n, m, float(eta), float(tol), int(max_iter),
          _stream_handle(stream, dev))


def birkhoff_eot_bwd(T, dT, a, dcost, eta: float = 1.0, stream=None) -> None:
    """eq (13) for the general problem: dcost = dL/dcost from the plan T and dT = dL/dT."""
    _plans(T, "T")
    B, n, m = T.shape
    sa = _marginal(a, "a", B, n)
    _plans(dT, "dT", B, n, m)
    _plans(dcost, "dcost", B, n, m)
    dev = _same_device(T, dT, a, dcost)
    _call("birkhoff_eot_bwd", dev, _p(T), _p(dT), _p(a), sa, _p(dcost), B, n, m, float(eta),
          _stream_handle(stream, dev))


def _streams(x, name, B=None, C=None, bf16=False):
    """Hidden states [B, 4, C]: float32, or bfloat16 / 16-bit bf16 patterns for the _bf16 entries."""
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    ok = (x.dtype in (torch.bfloat16, torch.int16, getattr(torch, "uint16", torch.int16))) if bf16 \
        else x.dtype == torch.float32
    if not ok:
        raise TypeError("%s has dtype %s" % (name, x.dtype))
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 3 or x.shape[1] != 4:
        raise ValueError("%s must be a contiguous GPU tensor of shape [B, 4, C], got %s" % (name, tuple(x.shape)))
    if B is not None and (x.shape[0] != B or x.shape[2] != C):
        raise ValueError("%s must have shape [%d, 4, %d], got %s" % (name, B, C, tuple(x.shape)))
    return x


def _fwd_mix(name, bf16, logits, x, T, dual, y, tol, max_iter, stream):
    torch = _torch()
    _mats(logits, "logits", torch.float32)
    B, n = logits.shape[0], logits.shape[1]
    _streams(x, "x", bf16=bf16)
    C = x.shape[2]
    _streams(x, "x", B, C, bf16)
    _streams(y, "y", B, C, bf16)
    _mats(T, "T", torch.float32, B, n)
    _vec(dual, "dual", B, n, torch.float32)
    dev = _same_device(logits, x, T, dual, y)
    _call(name, dev, _p(logits), _p(x), _p(T), _p(dual), _p(y), B, n, C, float(tol), int(max_iter),
          _stream_handle(stream, dev))


def birkhoff_fwd_mix(logits, x, T, dual, y, tol: float = 1e-6, max_iter: int = 50, stream=None) -> None:
    """Projection of logits [B,4,4] fused with y = T x for hidden states x [B,4,C] (fp32)."""
    _fwd_mix("birkhoff_fwd_mix", False, logits, x, T, dual, y, tol, max_iter, stream)


def birkhoff_fwd_mix_bf16(logits, x, T, dual, y, tol: float = 1e-6, max_iter: int = 50, stream=None) -> None:
    """As birkhoff_fwd_mix with bf16 hidden states x and y (fp32 logits, T, dual)."""
    _fwd_mix("birkhoff_fwd_mix_bf16", True, logits, x, T, dual, y, tol, max_iter, stream)


def _mix_bwd(name, bf16, T, x, dy, dx, dH, stream):
    torch = _torch()
    _mats(T, "T", torch.float32)
    B, n = T.shape[0], T.shape[1]
    _streams(x, "x", bf16=bf16)
    C = x.shape[2]
    _streams(x, "x", B, C, bf16)
    _streams(dy, "dy", B, C, bf16)
    _streams(dx, "dx", B, C, bf16)
    _mats(dH, "dH", torch.float32, B, n)
    dev = _same_device(T, x, dy, dx, dH)
    _call(name, dev, _p(T), _p(x), _p(dy), _p(dx), _p(dH), B, n, C, _stream_handle(stream, dev))


def birkhoff_mix_bwd(T, x, dy, dx, dH, stream=None) -> None:
    """Backward of y = T x and of the projection: dx = T^T dy, dH by eq (13) from dT = dy x^T (fp32)."""
    _mix_bwd("birkhoff_mix_bwd", False, T, x, dy, dx, dH, stream)


def birkhoff_mix_bwd_bf16(T, x, dy, dx, dH, stream=None) -> None:
    """As birkhoff_mix_bwd with bf16 hidden states x, dy and dx."""
    _mix_bwd("birkhoff_mix_bwd_bf16", True, T, x, dy, dx, dH, stream)


# ------------------------------------------------------- allocating helpers

def project(logits, tol: float = 1e-6, max_iter: int = 50, stream=None):
    """Allocate outputs and run the forward pass. Returns (T, dual); bf16 input gives bf16 T."""
    torch = _torch()
    B, n = logits.shape[0], logits.shape[1]
    dual = torch.empty((B, n), dtype=torch.float32, device=logits.device)
    T = torch.empty_like(logits, memory_format=torch.contiguous_format)
    if logits.dtype == torch.float32:
        birkhoff_fwd(logits, T, dual, tol, max_iter, stream)
    else:
        birkhoff_fwd_bf16(logits, T, dual, tol, max_iter, stream)
    return T, dual


def project_bwd(logits, dual, dT, stream=None):
    """Allocate dH and run the backward pass."""
    torch = _torch()
    dH = torch.empty_like(dT, memory_format=torch.contiguous_format)
    if logits.dtype == torch.float32:
        birkhoff_bwd(logits, dual, dT, dH, stream)
    else:
        birkhoff_bwd_bf16(logits, dual, dT, dH, stream)
    return dH


def project_fwd_bwd(logits, dT, tol: float = 1e-6, max_iter: int = 50, stream=None):
    """Allocate outputs and run forward + backward in one launch. Returns (T, dual, dH)."""
    torch = _torch()
    B, n = logits.shape[0], logits.shape[1]
    dual = torch.empty((B, n), dtype=torch.float32, device=logits.device)
    T = torch.empty_like(logits, memory_format=torch.contiguous_format)
    dH = torch.empty_like(dT, memory_format=torch.contiguous_format)
    if logits.dtype == torch.float32:
        birkhoff_fwd_bwd(logits, dT, T, dual, dH, tol, max_iter, stream)
    else:
        birkhoff_fwd_bwd_bf16(logits, dT, T, dual, dH, tol, max_iter, stream)
    return T, dual, dH


def sinkhorn(logits, iters: int = 20, stream=None):
    T = _torch().empty_like(logits, memory_format=_torch().contiguous_format)
    sinkhorn_fwd(logits, T, iters, stream)
    return T


def eot_plan(cost, a, b, eta: float = 1.0, tol: float = 1e-6, max_iter: int = 50, with_iters: bool = False,
             stream=None):
    """Allocate outputs and solve the general problems. Returns (T, dual) or (T, dual, iters)."""
    torch = _torch()
    B, n, m = cost.shape
    T = torch.empty((B, n, m), dtype=torch.float32, device=cost.device)
    dual = torch.empty((B, m), dtype=torch.float32, device=cost.device)
    iters = torch.empty((B,), dtype=torch.int32, device=cost.device) if with_iters else None
    birkhoff_eot_fwd(cost, a, b, T, dual, iters, eta, tol, max_iter, stream)
    return (T, dual, iters) if with_iters else (T, dual)


def eot_plan_bwd(T, dT, a, eta: float = 1.0, stream=None):
    """Allocate dcost and run eq (13)."""
    dcost = _torch().empty_like(T)
    birkhoff_eot_bwd(T, dT, a, dcost, eta, stream)
    return dcost


def project_mix(logits, x, tol: float = 1e-6, max_iter: int = 50, stream=None):
    """Project logits [B,4,4] and mix hidden states x [B,4,C]: returns (T, dual, y)."""
    torch = _torch()
    B, n = logits.shape[0], logits.shape[1]
    T = torch.empty((B, n, n), dtype=torch.float32, device=logits.device)
    dual = torch.empty((B, n), dtype=torch.float32, device=logits.device)
    y = torch.empty_like(x)
    if x.dtype == torch.float32:
        birkhoff_fwd_mix(logits, x, T, dual, y, tol, max_iter, stream)
    else:
        birkhoff_fwd_mix_bf16(logits, x, T, dual, y, tol, max_iter, stream)
    return T, dual, y


def project_mix_bwd(T, x, dy, stream=None):
    """Backward of project_mix: returns (dH, dx)."""
    torch = _torch()
    dH = torch.empty_like(T)
    dx = torch.empty_like(x)
    if x.dtype == torch.float32:
        birkhoff_mix_bwd(T, x, dy, dx, dH, stream)
    else:
        birkhoff_mix_bwd_bf16(T, x, dy, dx, dH, stream)
    return dH, dx


def _autograd_function():
    torch = _torch()

    class BirkhoffProjection(torch.autograd.Function):
        """T = proj_KL(exp(logits)) onto B_n with the implicit (eq 13) backward.

        No Newton iterates are kept.  The backward is computed by the kernels (not
        from differentiable torch operations), so it is once differentiable: a
        second derivative through it raises.  fp32 saves the output T and differentiates
        from it (birkhoff_bwd_from_T: the pages' backward from T* and G, 192 bytes
        per 4x4 projection and no exponentials, 6 % faster than recomputing T);
        bf16 storage saves (logits, dual) and recomputes T in fp32, since a
        bf16-rounded T would carry its rounding into Delta.
        """

        @staticmethod
        def forward(ctx, logits, tol: float = 1e-6, max_iter: int = 50):
            logits = logits.contiguous()
            T, dual = project(logits, tol, max_iter)
            if logits.dtype == torch.float32:
                ctx.save_for_backward(T)
            else:
                ctx.save_for_backward(logits, dual)
            return T

        @staticmethod
        @torch.autograd.function.once_differentiable
        def backward(ctx, dT):
            saved = ctx.saved_tensors
            dT = dT.contiguous()
            if len(saved) == 1:
                (T,) = saved
                dH = torch.empty_like(dT, memory_format=torch.contiguous_format)
                birkhoff_bwd_from_T(T, dT, dH)
                return dH, None, None
            logits, dual = saved
            return project_bwd(logits, dual, dT), None, None

    class EntropicOT(torch.autograd.Function):
        """Plan of the entropic OT problem with cost `cost` and fixed marginals a, b,
        differentiable in the cost by eq (13).  Saves (T, a)."""

        @staticmethod
        def forward(ctx, cost, a, b, eta: float = 1.0, tol: float = 1e-6, max_iter: int = 50):
            T, _ = eot_plan(cost.contiguous(), a, b, eta, tol, max_iter)
            ctx.save_for_backward(T, a)
            ctx.eta = eta
            return T

        @staticmethod
        @torch.autograd.function.once_differentiable
        def backward(ctx, dT):
            T, a = ctx.saved_tensors
            return eot_plan_bwd(T, dT.contiguous(), a, ctx.eta), None, None, None, None, None

    class ProjectMix(torch.autograd.Function):
        """y = proj_KL(exp(logits)) x per token (the mHC residual mixing H_res x),
        differentiable in both the logits (eq 13) and x.  Saves (T, x)."""

        @staticmethod
        def forward(ctx, logits, x, tol: float = 1e-6, max_iter: int = 50):
            T, _, y = project_mix(logits.contiguous(), x.contiguous(), tol, max_iter)
            ctx.save_for_backward(T, x)
            return y

        @staticmethod
        @torch.autograd.function.once_differentiable
        def backward(ctx, dy):
            T, x = ctx.saved_tensors
            dH, dx = project_mix_bwd(T, x.contiguous(), dy.contiguous())
            return dH, dx, None, None

    return {"BirkhoffProjection": BirkhoffProjection, "EntropicOT": EntropicOT, "ProjectMix": ProjectMix}


class _LazyFunction:
    _fns = None

    def __init__(self, name):
        self._name = name

    def __getattr__(self, item):
        if _LazyFunction._fns is None:
            _LazyFunction._fns = _autograd_function()
        return getattr(_LazyFunction._fns[self._name], item)


BirkhoffProjection = _LazyFunction("BirkhoffProjection")
EntropicOT = _LazyFunction("EntropicOT")
ProjectMix = _LazyFunction("ProjectMix")
