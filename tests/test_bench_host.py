"""Host-side logic of bench.py (no GPU): the one-GPU guard, workload lookup and
the roofline record built from committed counter summaries."""
import importlib.util
import json
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]


def run_bench(*args):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_workload_is_refused():
    r = run_bench("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "unknown workload" in r.stderr


def test_roofline_record(tmp_path, monkeypatch):
    bench = load_bench()
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    (tmp_path / "profiles").mkdir()
    prof = {"kernel_digest": "abc", "bytes_per_launch": {"k": 1.5e8},
            "valu_active_per_launch": {"k": 0.5 * 256 * 1e-4 * 2.4e9},
            "valu_insts_per_launch": {"k": 0.25 * 256 * 1e-4 * 2.4e9}}
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(prof))
    r = bench.roofline("w", "k", 8e8, 0.1, "abc")      # 8e8 bytes in 0.1 ms = 8 TB/s
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 8000.0) < 1e-9 and abs(r["frac"] - 1.0) < 1e-12
    assert r["traffic"] == 1.5e8
    assert abs(r["valu_busy"] - 0.5) < 1e-12
    assert r["valu"]["unit"] == "lane-instructions/s" and abs(r["valu"]["frac"] - 0.25) < 1e-12
    assert abs(r["valu"]["peak"] - 256 * 64 * 2.4e9) < 1.0
    # counters taken on other kernel sources are not used
    r2 = bench.roofline("w", "k", 8e8, 0.1, "other")
    assert r2["traffic"] is None and "valu_busy" not in r2 and "valu" not in r2
