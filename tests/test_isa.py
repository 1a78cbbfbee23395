"""Code-generation checks on the gfx950 assembly of the kernels (CPU only: hipcc
cross-compiles).  They pin properties the measured performance depends on:
every matrix / dual store is non-temporal, the n = 4 kernels keep their
occupancy and spill nothing, the n = 8 kernels keep three waves per SIMD without
spilling, and the
general-OT kernels spill nothing and stream their stores too."""
import re
import shutil
import subprocess

import pytest

from birkhoff_projection_amd import build as hipbuild

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not hipbuild.os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def compile_asm(tmp_path_factory, source):
    out = tmp_path_factory.mktemp("isa") / (source + ".s")
    cmd = [hipbuild.hipcc(), "--offload-arch=%s" % hipbuild.ARCH, "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", str(hipbuild.ROOT / "include"), "-I", str(hipbuild.CSRC),
           "--cuda-device-only", "-S", str(hipbuild.CSRC / source), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return compile_asm(tmp_path_factory, "birkhoff.hip")


@pytest.fixture(scope="module")
def asm_mix(tmp_path_factory):
    return compile_asm(tmp_path_factory, "mix.hip")


@pytest.fixture(scope="module")
def asm_eot(tmp_path_factory):
    """The general-OT kernels for n = 4 and 5 rows (every column count)."""
    return compile_asm(tmp_path_factory, "eot_rows_45.hip")


def kernels(asm):
    """{mangled kernel name: (body text, vgprs, scratch bytes, occupancy)}"""
    out = {}
    for m in re.finditer(r"^(_ZN4birk\w+):.*?\n(.*?)^; Occupancy: (\d+)", asm, flags=re.M | re.S):
        body = m.group(2)
        vgpr = int(re.search(r"; TotalNumVgprs: (\d+)", body).group(1))
        scratch = int(re.search(r"; ScratchSize: (\d+)", body).group(1))
        out[m.group(1)] = (body, vgpr, scratch, int(m.group(3)))
    return out


def test_all_global_stores_are_non_temporal(asm):
    """Streaming stores everywhere, but for the gathering forward's per-lane T of a
    gathered matrix (one 64-byte fp32 or 32-byte bf16 piece among lines written
    by other waves), which is cached so that the L2 merges it (4 or 2 stores)."""
    ks = kernels(asm)
    assert ks
    for name, (body, *_rest) in ks.items():
        cached = [line for line in re.findall(r"^\s+global_store_dwordx4.*$", body, flags=re.M)
                  if not line.rstrip().endswith(" nt")]
        if "newton_fwd_gather_kernel" in name:
            assert len(cached) == (4 if "gather_kernelIf" in name else 2), (name, cached)
        else:
            assert not cached, (name, cached)


def test_n4_kernels_occupancy_and_no_spills(asm):
    ks = kernels(asm)
    # the gathering forward that the plain entry point runs keeps seven waves per SIMD;
    # its statistics variant (iteration and fallback counts) six
    want = {"newton_fwd_gather_kernelIfLb0E": 7, "newton_fwd_gather_kernelIfLb1E": 6,
            "fused_fwd_bwd_kernelILi4Ef": 6, "implicit_bwd_kernelILi4Ef": 7}
    for key, occ in want.items():
        hits = [v for k, v in ks.items() if key in k]
        assert hits, key
        for _, vgpr, scratch, o in hits:
            assert scratch == 0 and o >= occ, (key, vgpr, scratch, o)


def test_n8_kernels_keep_three_waves_without_spills(asm):
    """At four waves per SIMD (128 VGPRs) the n = 8 fused kernel spilled 104 bytes
    per lane, which showed up as 0.5 GB of extra HBM traffic per launch; three
    waves and no scratch measured 18 % faster."""
    ks = kernels(asm)
    hits = [v for k, v in ks.items() if "ILi8E" in k and "sinkhorn" not in k]
    assert hits
    for _, vgpr, scratch, o in hits:
        assert o >= 3 and scratch == 0, (vgpr, scratch, o)


def test_no_kernel_uses_scratch(asm):
    for name, (_, vgpr, scratch, _o) in kernels(asm).items():
        assert scratch == 0, (name, vgpr, scratch)


def test_eot_kernels_stream_and_do_not_spill(asm_eot):
    ks = kernels(asm_eot)
    assert len(ks) == 2 * 7 * 3   # n = 4, 5; m = 2..8; forward with and without counts, backward
    for name, (body, vgpr, scratch, occ) in ks.items():
        assert scratch == 0, (name, vgpr)
        for line in re.findall(r"^\s+global_store_dword(?:x4)?\s.*$", body, flags=re.M):
            assert line.rstrip().endswith(" nt"), (name, line)
    small = [v for k, v in ks.items() if "eot_fwd_kernelILi4ELi4E" in k]
    assert small and all(o >= 4 for _, _, _, o in small)


SCALAR_WRITES = re.compile(r"^\s+s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)",
                           re.M)


def test_no_kernel_writes_through_the_scalar_cache(asm, asm_eot, asm_mix):
    """Every store and atomic of the library is a vector-memory instruction: no
    scalar-memory stores, atomics, write-backs or discards in any kernel."""
    for text in (asm, asm_eot, asm_mix):
        assert not SCALAR_WRITES.findall(text)


def test_mix_kernels_stream_and_do_not_spill(asm_mix):
    ks = kernels(asm_mix)
    assert len(ks) == 4
    for name, (body, vgpr, scratch, occ) in ks.items():
        assert scratch == 0 and occ >= 3, (name, vgpr, occ)
        for line in re.findall(r"^\s+global_store_dwordx4.*$", body, flags=re.M):
            assert line.rstrip().endswith(" nt"), (name, line)
