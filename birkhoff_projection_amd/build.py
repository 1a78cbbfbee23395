"""Build libbirkhoff.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m birkhoff_projection_amd.build [--resource-usage]

The library is written next to this file; the Python binding loads it from
there.  All device code is compiled with packed-FP32 instruction selection
turned off (the -packed-fp32-ops target feature), for every kernel.
"""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libbirkhoff.so"
SOURCES = [CSRC / "birkhoff.hip"]
ARCH = "gfx950"


def kernel_source_digest() -> str:
    """Short hash of every device / ABI source file; identifies which kernels a
    profile was taken on."""
    import hashlib
    h = hashlib.sha256()
    for p in sorted(list(CSRC.glob("*")) + [ROOT / "include" / "birkhoff.h"]):
        if p.is_file():
            h.update(p.name.encode())
            h.update(p.read_bytes())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbirkhoff)")


def command(out: pathlib.Path, resource_usage: bool = False) -> list:
    cmd = [hipcc(), "--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-I", str(ROOT / "include"), "-I", str(CSRC)]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [str(s) for s in SOURCES] + ["-o", str(out)]
    return cmd


def build(resource_usage: bool = False, quiet: bool = True) -> pathlib.Path:
    """Compile every HIP source into libbirkhoff.so (always recompiles)."""
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    r = subprocess.run(command(tmp, resource_usage), capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and not quiet:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, quiet=False)
    print(LIB)
