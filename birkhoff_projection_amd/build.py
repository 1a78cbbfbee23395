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
SOURCES = sorted(CSRC.glob("*.hip"))
ARCH = "gfx950"


def _code_only(text: str) -> str:
    """C/C++ source with comments, trailing blanks and empty lines removed (the
    sources hold no string literal containing a comment marker)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_digest() -> str:
    """Short hash of the code (comments excluded) of every device / ABI source
    file; identifies which kernels a profile was taken on."""
    import hashlib
    h = hashlib.sha256()
    for p in sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.hpp")) + [ROOT / "include" / "birkhoff.h"]):
        h.update(p.name.encode())
        h.update(_code_only(p.read_text()).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbirkhoff)")


def flags(resource_usage: bool = False) -> list:
    f = ["--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", str(ROOT / "include"), "-I", str(CSRC)]
    if resource_usage:
        f += ["-Rpass-analysis=kernel-resource-usage"]
    return f


# the host pass does not know the packed-fp32 target feature and says so
_NOISE = "is not a recognized feature for this target"


def _errors(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if _NOISE not in l)


def build(resource_usage: bool = False, quiet: bool = True) -> pathlib.Path:
    """Compile every HIP source into libbirkhoff.so (always recompiles).  The
    translation units are compiled in parallel, then linked."""
    tag = "tmp%d" % os.getpid()
    objs = [LIB.with_name("%s.%s.o" % (src.stem, tag)) for src in SOURCES]
    procs = [subprocess.Popen([hipcc()] + flags(resource_usage) + ["-c", str(src), "-o", str(obj)],
                              stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
             for src, obj in zip(SOURCES, objs)]
    errs, failed = [], False
    for pr in procs:
        _, err = pr.communicate()
        failed |= pr.returncode != 0
        errs.append(_errors(err))
    tmp = LIB.with_suffix(".so." + tag)
    try:
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
        r = subprocess.run([hipcc(), "--offload-arch=%s" % ARCH, "-shared", "-fPIC"] + [str(o) for o in objs]
                           + ["-o", str(tmp)], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + _errors(r.stderr))
        err = "\n".join(errs + [_errors(r.stderr)]).strip()
        if err and not quiet:
            print(err, file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        for o in objs + [tmp]:
            if o.exists():
                o.unlink()
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, quiet=False)
    print(LIB)
