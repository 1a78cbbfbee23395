"""Host-only sanitizer builds: the float64 oracle (oracle/oracle.c) and the C
ABI's argument validation (csrc/abi_checks.hpp) compiled by gcc / g++ with the
address and undefined-behaviour sanitizers, and run by the drivers in
tests/sanitize/ on small seeded inputs, edge sizes and every rejected
argument.  Any invalid access or undefined operation aborts the driver."""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run_driver(exe: pathlib.Path, want: str):
    env = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1",
           "PATH": "/usr/bin:/bin"}
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert want in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", *SAN, "-Wall", "-Wno-unknown-pragmas",
           str(ROOT / "oracle" / "oracle.c"), str(ROOT / "tests" / "sanitize" / "oracle_driver.c"), "-lm",
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    run_driver(exe, "oracle driver: ok")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_validation_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-std=c++17", *SAN, "-Wall", "-I", str(ROOT / "include"),
           "-I", str(ROOT / "birkhoff_projection_amd" / "csrc"),
           str(ROOT / "tests" / "sanitize" / "abi_driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    run_driver(exe, "abi driver: ok")
