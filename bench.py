#!/usr/bin/env python3
"""Benchmark: 4x4 Birkhoff projections per second (forward + backward, fp32) on one MI355X.

One step = the whole hot path over one batch: the Newton projection and the
implicit backward for every matrix of the workload.  The default workload is
the training-shaped mHC pass -- B = 16 sequences x 4096 tokens x 32 layers =
2,097,152 matrices of 4x4 fp32 logits H = N(0, 0.5^2) + 2I with upstream
dL/dT = N(0, 0.1^2), tol 1e-6 -- whose forward and backward are fused.  The
timed step is therefore one birkhoff_fwd_bwd launch (--path fused, default);
--path separate times birkhoff_fwd followed by birkhoff_bwd instead.  Either
way the other form is timed too and reported under "other_path", and the
timed step is also captured into a HIP graph and replayed ("graph_replay":
the same kernels without the host's launch work between them, which is what
decides the small, launch-bound workload).

Inputs are generated on the host from fixed seeds and copied to HBM before
anything is timed.  Two complete input/output sets alternate between steps, so
that a step never finds the previous step's data in the 256 MB last-level
cache.  Before the counted warm-up, steps run back to back for --settle-ms of
wall time (400 ms by default), so that the engine clock has left its idle
level whatever --warmup is.  The timed region is `--steps` back-to-back steps
between two HIP events on the stream the kernels run on; `value` is
B / (time per step).  `clock` records the settle phase and the engine clock
that a probe kernel measures right behind the timed region, on the same
stream (shader-clock cycles per tick of the constant-rate counter).

The roofline figure is for the kernel with the longer average launch time
(the fused kernel is the only one of its step); see roofline() for the VALU
figure that accompanies it when counters for the same kernel sources exist.  Each separate kernel's
average launch time is measured as `--steps` back-to-back launches of that
kernel alone (alternating the two sets) between two HIP events on the same
stream -- events between the two kernels of a step would themselves add gaps.
`achieved` divides the kernel's algorithmic bytes per launch (each input read
once, each output written once) by that time.  `traffic` is the HBM traffic
per launch that rocprofv3's FETCH_SIZE / WRITE_SIZE counters measured for the
same kernel sources (profiles/traffic_<workload>.json), or null when the
kernels have changed since.

The CPU baseline is the float64 oracle timed on a bounded sample of the same
workload on this host's cores (all of them, and one), with the CPU model and
the time of its parts (the Sinkhorn reference to 1e-13, the Newton cross-check,
the backward) on the same sample.

    python bench.py [--gpus 1] [--steps 200] [--warmup 300] [--workload train] [--path fused|separate]
"""
from __future__ import annotations

import argparse
import json
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s
METRIC = "4x4 Birkhoff projections/sec (fwd+bwd, fp32) on 1 MI355X; % HBM roofline"


CLOCK_HZ = 2.4e9   # MI355X peak engine clock
N_CU = 256


def _profile(workload: str, digest: str):
    p = ROOT / "profiles" / ("traffic_%s.json" % workload)
    if not p.exists():
        return {}
    d = json.loads(p.read_text())
    return d if d.get("kernel_digest") == digest else {}


def measured_traffic(workload: str, kernel: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    return _profile(workload, digest).get("bytes_per_launch", {}).get(kernel)


def roofline(workload: str, kernel: str, nbytes: float, ms: float, digest: str) -> dict:
    """The dominant kernel against the HBM roofline: algorithmic bytes per launch
    over the launch time, against 8 TB/s.  When committed counters exist for the
    same kernel sources, `valu_busy` adds AMD's VALUBusy measure for the same
    launch time -- SQ_ACTIVE_INST_VALU / (CUs x cycles), cycles = time x 2.4 GHz --
    which an issue-saturated fp32 FMA loop drives to about 0.9 on this chip, and
    `valu` the launch's vector instructions (SQ_INSTS_VALU x 64 lanes) per second
    against the fp32 issue peak of 256 CUs x 64 lanes x 2.4 GHz."""
    hbm = nbytes / (ms * 1e-3) / 1e9
    out = {"bound": "hbm", "kernel": kernel, "achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": hbm / HBM_PEAK_GBS, "traffic": measured_traffic(workload, kernel, digest),
           "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms}
    prof = _profile(workload, digest)
    active = prof.get("valu_active_per_launch", {}).get(kernel)
    if active is not None:
        out["valu_busy"] = active / N_CU / (ms * 1e-3 * CLOCK_HZ)
    insts = prof.get("valu_insts_per_launch", {}).get(kernel)
    if insts is not None:
        # the same launch against the fp32 VALU issue peak: every CU issues one
        # 64-lane vector instruction per cycle (the 157.3 TFLOP/s figure also counts
        # packed two-wide FMAs, which this code does not use)
        peak = N_CU * 64 * CLOCK_HZ
        achieved = insts * 64 / (ms * 1e-3)
        out["valu"] = {"achieved": achieved, "peak": peak, "unit": "lane-instructions/s", "frac": achieved / peak}
    return out


def settle(step, sets, ms: float):
    """Runs `step` back to back (alternating the two sets) for `ms` milliseconds of
    wall time before the counted warm-up.  The engine clock ramps up over tens of
    milliseconds of load after idle (the first ~100 launches of the 86 us fused
    step average 122 us), so a short counted warm-up alone would time the
    VALU-bound kernels on a low clock.  Returns the number of steps run."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(sets[i % 2])
            i += 1
        torch.cuda.synchronize()
    return i


def timed_steps(fn, sets, K: int, stream, probe=None) -> float:
    """K launches of fn (alternating the two sets) between two HIP events on
    `stream`; returns ms per launch.  With `probe` (a ClockProbe) the clock probe
    is enqueued right behind the end event, so that it measures the engine clock
    the timed launches ended on (it runs after the region, outside its time)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        fn(sets[i % 2])
    e1.record(stream)
    if probe is not None:
        probe.launch(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def per_kernel_time(fn, sets, K: int, stream, settle_ms: float, probe, clocks: dict, name: str) -> float:
    """A per-kernel figure: `fn` alone, back to back for a quarter of the settle
    time (at least 20 ms) so that the engine clock settles on that kernel's own
    load, then K timed launches (timed_steps); the clock after them goes into
    clocks[name].  Returns ms per launch."""
    settle(fn, sets, max(20.0, settle_ms / 4))
    ms = timed_steps(fn, sets, K, stream, probe)
    clocks[name] = round(probe.mhz(), 1)
    return ms


def clock_report(settle_steps, settle_ms, probe):
    """The settle phase and the engine clock measured right after the timed region
    (shader-clock cycles per constant-rate tick, birkhoff_clock_probe)."""
    return {"settle_ms": settle_ms, "settle_steps": settle_steps,
            "mhz_after_timed_region": round(probe.mhz(), 1), "peak_mhz": CLOCK_HZ / 1e6,
            "mhz_after_per_kernel": {}}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_seconds(kind: str, key: str, Bs: int) -> float:
    """Wall time of the float64 oracle on the first Bs items of a workload, on the
    threads OpenMP gives it: "proj" the certified projection and, where the
    workload has an upstream gradient, the eq (13) backward; "eot" the certified
    general plan and its backward; "mix" the projection, y = T x, its backward and
    eq (13)."""
    import oracle
    from birkhoff_projection_amd import workloads as W
    if kind == "proj":
        w = W.WORKLOADS[key]
        H = W.decode_f64(W.make_logits(w, B=Bs))
        G = None if w.upstream is None else W.decode_f64(W.make_upstream(w, B=Bs))
        t0 = time.perf_counter()
        T, _, _ = oracle.project(H, sk_cap=w.sk_cap)
        if G is not None:
            oracle.bwd(T, G)
        return time.perf_counter() - t0
    if kind == "eot":
        w = W.EOT_WORKLOADS[key]
        M, a, b = W.make_eot(w, B=Bs)
        G = W.make_eot_upstream(w, B=Bs)
        M, a, b, G = (x.astype("float64") for x in (M, a, b, G))
        t0 = time.perf_counter()
        T, _, _ = oracle.eot_project(M, a, b, w.eta, sk_cap=w.sk_cap)
        oracle.eot_bwd(T, G, a, b, w.eta)
        return time.perf_counter() - t0
    w = W.MIX_WORKLOADS[key]
    H, x, dy = W.make_mix(w, B=Bs)
    H, x, dy = H.astype("float64"), W.decode_f64(x), W.decode_f64(dy)
    t0 = time.perf_counter()
    T, _, _ = oracle.project(H)
    oracle.mix(T, x)
    _, dT = oracle.mix_bwd(T, x, dy)
    oracle.bwd(T, dT)
    return time.perf_counter() - t0


ONE_CORE_SCRIPT = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import bench, oracle
print(json.dumps({"seconds": bench.oracle_seconds(sys.argv[2], sys.argv[3], int(sys.argv[4])),
                  "threads": oracle.threads()}))
"""


def one_core_baseline(kind: str, key: str, n_items: int, per_item_s: float, unit: str = "matrices",
                      target_s: float = 5.0):
    """The same oracle on one core: a child process with OMP_NUM_THREADS=1 on a
    prefix sized to about target_s seconds from per_item_s, the one-core time
    per item that the all-core run implies."""
    import os
    import subprocess
    Bs = int(min(n_items, max(256, target_s / max(per_item_s, 1e-9))))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", ONE_CORE_SCRIPT, str(ROOT), kind, key, str(Bs)], env=env,
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1] if r.stderr.strip() else "failed"}
    d = json.loads(r.stdout.strip().splitlines()[-1])
    return {"value": Bs / d["seconds"], "cores": d["threads"],
            "sample": "the first %d %s, %.1f s wall" % (Bs, unit, d["seconds"])}


def cpu_baseline(w, target_s: float = 10.0):
    """The float64 oracle (reference projection + eq (13) backward) on a bounded
    sample of the workload, on this host's cores."""
    import oracle
    from birkhoff_projection_amd import workloads as W

    fwd_only = w.upstream is None

    def run(Bs):
        H = W.decode_f64(W.make_logits(w, B=Bs))
        G = None if fwd_only else W.decode_f64(W.make_upstream(w, B=Bs))
        t0 = time.perf_counter()
        T, _, _ = oracle.project(H, sk_cap=w.sk_cap)
        if not fwd_only:
            oracle.bwd(T, G)
        return time.perf_counter() - t0

    probe = 8192
    dt = run(probe)
    Bs = int(min(w.B, max(probe, probe * target_s / max(dt, 1e-6))))
    dt = run(Bs)
    # the parts of the same work, on the same prefix and cores: the Sinkhorn
    # reference to 1e-13 (capped) and the float64 Newton cross-check that
    # oracle.project runs for every matrix, and the backward
    H = W.decode_f64(W.make_logits(w, B=Bs))
    parts = {}
    t0 = time.perf_counter()
    oracle.sinkhorn_tol(H, tol=1e-13, cap=w.sk_cap)
    parts["sinkhorn_to_1e-13_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    T, _, _ = oracle.newton(H, tol=1e-13, max_iter=500)
    parts["newton_cross_check_s"] = time.perf_counter() - t0
    if not fwd_only:
        G = W.decode_f64(W.make_upstream(w, B=Bs))
        t0 = time.perf_counter()
        oracle.bwd(T, G)
        parts["eq13_backward_s"] = time.perf_counter() - t0
    return {"value": Bs / dt, "unit": "projections/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "the first %d matrices of the same seeded workload (%s), float64: Sinkhorn to 1e-13 "
                      "(cap %d sweeps) with a Newton cross-check%s; %.1f s wall"
                      % (Bs, "all of it" if Bs == w.B else "a prefix", w.sk_cap,
                         "" if fwd_only else ", then the eq (13) backward", dt),
            "cpu_model": cpu_model(), "parts": parts,
            "one_core": one_core_baseline("proj", w.key, w.B, dt / Bs * oracle.threads())}


def eot_cpu_baseline(w, target_s: float = 10.0):
    """The float64 oracle for the general problem (certified plan + eq (13)
    backward) on a bounded sample of the workload, on this host's cores."""
    import oracle
    from birkhoff_projection_amd import workloads as W

    probe = 8192
    dt = oracle_seconds("eot", w.key, probe)
    Bs = int(min(w.B, max(probe, probe * target_s / max(dt, 1e-6))))
    dt = oracle_seconds("eot", w.key, Bs)
    return {"value": Bs / dt, "unit": "problems/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "the first %d problems of the same seeded workload (%s), float64: Sinkhorn to 1e-13 "
                      "with a Newton cross-check, then the eq (13) backward; %.1f s wall"
                      % (Bs, "all of it" if Bs == w.B else "a prefix", dt),
            "cpu_model": cpu_model(),
            "one_core": one_core_baseline("eot", w.key, w.B, dt / Bs * oracle.threads(), "problems")}


def eot_report(w, args, dev):
    """A general entropic-OT workload: the step is birkhoff_eot_fwd then
    birkhoff_eot_bwd (the backward at the forward's plan)."""
    import torch

    import birkhoff_projection_amd as bp
    from birkhoff_projection_amd import build as hipbuild
    from birkhoff_projection_amd import workloads as W

    B, n, m = w.B, w.n, w.m
    M, a, b = W.make_eot(w)
    G = W.make_eot_upstream(w)
    sets = []
    for _ in range(2):
        st = {k: torch.from_numpy(v).to(dev) for k, v in (("M", M), ("a", a), ("b", b), ("G", G))}
        st["T"] = torch.empty((B, n, m), dtype=torch.float32, device=dev)
        st["D"] = torch.empty((B, n, m), dtype=torch.float32, device=dev)
        st["dual"] = torch.empty((B, m), dtype=torch.float32, device=dev)
        sets.append(st)
    del M, a, b, G
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def run_fwd(s):
        bp.birkhoff_eot_fwd(s["M"], s["a"], s["b"], s["T"], s["dual"], None, w.eta, w.tol, w.max_iter, stream)

    def run_bwd(s):
        bp.birkhoff_eot_bwd(s["T"], s["G"], s["a"], s["D"], w.eta, stream)

    def step(s):
        run_fwd(s)
        run_bwd(s)

    def timed(fn, K, probe=None):
        return timed_steps(fn, sets, K, stream, probe)

    def kernel_time(fn, name):
        return per_kernel_time(fn, sets, args.steps, stream, args.settle_ms, probe, clock["mhz_after_per_kernel"], name)

    settle_steps = settle(step, sets, args.settle_ms)
    probe = bp.ClockProbe(dev)
    for i in range(args.warmup):
        step(sets[i % 2])
    torch.cuda.synchronize()
    K = args.steps
    ms_step = timed(step, K, probe)
    clock = clock_report(settle_steps, args.settle_ms, probe)
    fwd_ms = kernel_time(run_fwd, "birkhoff_eot_fwd")
    bwd_ms = kernel_time(run_bwd, "birkhoff_eot_bwd")
    iters = torch.empty(B, dtype=torch.int32, device=dev)
    st = sets[0]
    bp.birkhoff_eot_fwd(st["M"], st["a"], st["b"], st["T"], st["dual"], iters, w.eta, w.tol, w.max_iter, stream)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    waves = it[: (B // 64) * 64].reshape(-1, 64)

    b_fwd = W.eot_bytes_per_problem(n, m, "fwd", w.shared) * B
    b_bwd = W.eot_bytes_per_problem(n, m, "bwd", w.shared) * B
    kern = {"birkhoff_eot_fwd": (fwd_ms, b_fwd), "birkhoff_eot_bwd": (bwd_ms, b_bwd)}
    dom = max(kern, key=lambda k: kern[k][0])
    d_ms, d_bytes = kern[dom]
    digest = hipbuild.kernel_source_digest()
    return {
        "metric": "%dx%d entropic OT plans/sec (fwd+bwd, fp32, general cost / marginals / eta) on 1 MI355X; "
                  "%% HBM roofline" % (n, m),
        "value": B / (ms_step * 1e-3), "unit": "problems/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (w.key, w.title), "B": B, "n": n, "m": m, "eta": w.eta,
                   "shared_marginals": w.shared, "passes": "fwd+bwd", "tol": w.tol, "max_iter": w.max_iter},
        "roofline": roofline(w.key, dom, d_bytes, d_ms, digest),
        "copy_ref": copy_reference(d_bytes, d_bytes / (d_ms * 1e-3) / 1e9, dev),
        "kernels_ms": {"birkhoff_eot_fwd": fwd_ms, "birkhoff_eot_bwd": bwd_ms},
        "kernels_hbm_frac": {k: v[1] / (v[0] * 1e-3) / 1e9 / HBM_PEAK_GBS for k, v in kern.items()},
        "newton": {"iterations_mean": float(it[it >= 0].mean()), "wave_max_mean": float(waves.max(1).mean()),
                   "unconverged": int((it < 0).sum())},
        "clock": clock,
        "kernel_digest": digest,
    }


def mix_cpu_baseline(w, target_s: float = 10.0):
    """The float64 oracle for the projection and its consumer (certified projection,
    y = T x, dx and dT, eq (13)) on a bounded sample of the workload's tokens."""
    import oracle
    from birkhoff_projection_amd import workloads as W

    probe = 256
    dt = oracle_seconds("mix", w.key, probe)
    Bs = int(min(w.B, max(probe, probe * target_s / max(dt, 1e-6))))
    dt = oracle_seconds("mix", w.key, Bs)
    return {"value": Bs / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "the first %d tokens of the same seeded workload (%s), float64: the certified projection, "
                      "y = T x, dx = T^T dy, dT = dy x^T and the eq (13) backward; %.1f s wall"
                      % (Bs, "all of it" if Bs == w.B else "a prefix", dt),
            "cpu_model": cpu_model(),
            "one_core": one_core_baseline("mix", w.key, w.B, dt / Bs * oracle.threads(), "tokens")}


def mix_report(w, args, dev):
    """The projection with its consumer: the step is birkhoff_fwd_mix (project the
    tokens' logits and mix their hidden states, y = T x) then birkhoff_mix_bwd (dx,
    and dH through eq (13))."""
    import torch

    import birkhoff_projection_amd as bp
    from birkhoff_projection_amd import build as hipbuild
    from birkhoff_projection_amd import workloads as W

    B, C = w.B, w.C
    H, x, dy = W.make_mix(w)

    def to_dev(a):
        t = torch.from_numpy(a).to(dev)
        return t.view(torch.bfloat16) if w.io == "bf16" else t

    sets = []
    for _ in range(2):
        st = {"H": torch.from_numpy(H).to(dev), "x": to_dev(x), "dy": to_dev(dy)}
        st["y"] = torch.empty_like(st["x"])
        st["dx"] = torch.empty_like(st["x"])
        st["T"] = torch.empty((B, 4, 4), dtype=torch.float32, device=dev)
        st["dual"] = torch.empty((B, 4), dtype=torch.float32, device=dev)
        st["dH"] = torch.empty((B, 4, 4), dtype=torch.float32, device=dev)
        sets.append(st)
    del H, x, dy
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    fwd = bp.birkhoff_fwd_mix_bf16 if w.io == "bf16" else bp.birkhoff_fwd_mix
    bwd = bp.birkhoff_mix_bwd_bf16 if w.io == "bf16" else bp.birkhoff_mix_bwd

    def run_fwd(s):
        fwd(s["H"], s["x"], s["T"], s["dual"], s["y"], w.tol, w.max_iter, stream)

    def run_bwd(s):
        bwd(s["T"], s["x"], s["dy"], s["dx"], s["dH"], stream)

    def step(s):
        run_fwd(s)
        run_bwd(s)

    def timed(fn, K, probe=None):
        return timed_steps(fn, sets, K, stream, probe)

    def kernel_time(fn, name):
        return per_kernel_time(fn, sets, args.steps, stream, args.settle_ms, probe, clock["mhz_after_per_kernel"], name)

    settle_steps = settle(step, sets, args.settle_ms)
    probe = bp.ClockProbe(dev)
    for i in range(args.warmup):
        step(sets[i % 2])
    torch.cuda.synchronize()
    K = args.steps
    ms_step = timed(step, K, probe)
    clock = clock_report(settle_steps, args.settle_ms, probe)
    fwd_ms = kernel_time(run_fwd, "birkhoff_fwd_mix")
    bwd_ms = kernel_time(run_bwd, "birkhoff_mix_bwd")
    # context only: the same product through torch's batched matmul on the stored T
    def run_torch(s):
        torch.matmul(s["T"].to(s["x"].dtype), s["x"], out=s["y"])
    torch_ms = timed(run_torch, max(10, K // 4))

    b_fwd = W.mix_bytes_per_token(C, w.io, "fwd") * B
    b_bwd = W.mix_bytes_per_token(C, w.io, "bwd") * B
    kern = {"birkhoff_fwd_mix": (fwd_ms, b_fwd), "birkhoff_mix_bwd": (bwd_ms, b_bwd)}
    dom = max(kern, key=lambda k: kern[k][0])
    d_ms, d_bytes = kern[dom]
    digest = hipbuild.kernel_source_digest()
    return {
        "metric": "mHC tokens/sec: 4x4 projection + residual mixing y = T x and its backward (C=%d, %s streams) "
                  "on 1 MI355X; %% HBM roofline" % (C, w.io),
        "value": B / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "%s: %s" % (w.key, w.title), "B": B, "C": C, "storage": w.io,
                   "passes": "fwd+bwd", "tol": w.tol, "max_iter": w.max_iter},
        "roofline": roofline(w.key, dom, d_bytes, d_ms, digest),
        "copy_ref": copy_reference(d_bytes, d_bytes / (d_ms * 1e-3) / 1e9, dev),
        "kernels_ms": {"birkhoff_fwd_mix": fwd_ms, "birkhoff_mix_bwd": bwd_ms},
        "kernels_hbm_frac": {k: v[1] / (v[0] * 1e-3) / 1e9 / HBM_PEAK_GBS for k, v in kern.items()},
        "torch_matmul_y_ms": torch_ms,
        "clock": clock,
        "kernel_digest": digest,
    }


def forward_only_report(w, args, dev):
    """A forward-only workload (the hard-conditioning one): the timed step is one
    birkhoff_fwd launch; the fixed 20-sweep Sinkhorn-Knopp kernel is timed on the
    same inputs, and both outputs are scored (Newton iteration histogram, the
    residual and the L1 marginal error of the blog post's accuracy metric, in
    float64)."""
    import torch

    import birkhoff_projection_amd as bp
    from birkhoff_projection_amd import build as hipbuild
    from birkhoff_projection_amd import workloads as W

    B, n = w.B, w.n
    Hs = W.make_logits(w)
    sets = [dict(H=torch.from_numpy(Hs).to(dev)) for _ in range(2)]
    for st in sets:
        st["T"] = torch.empty_like(st["H"])
        st["S"] = torch.empty_like(st["H"])
        st["dual"] = torch.empty((B, n), dtype=torch.float32, device=dev)
    del Hs
    stream = torch.cuda.current_stream(dev)

    def run_fwd(st):
        bp.birkhoff_fwd(st["H"], st["T"], st["dual"], w.tol, w.max_iter, stream)

    def run_sk(st):
        bp.sinkhorn_fwd(st["H"], st["S"], 20, stream)

    def timed(fn, K, probe=None):
        return timed_steps(fn, sets, K, stream, probe)

    def kernel_time(fn, name):
        return per_kernel_time(fn, sets, args.steps, stream, args.settle_ms, probe, clock["mhz_after_per_kernel"], name)

    settle_steps = settle(run_fwd, sets, args.settle_ms)
    probe = bp.ClockProbe(dev)
    for i in range(args.warmup):
        run_fwd(sets[i % 2])
    K = args.steps
    ms = timed(run_fwd, K, probe)
    clock = clock_report(settle_steps, args.settle_ms, probe)
    ms_sk = kernel_time(run_sk, "sinkhorn_fwd")
    st = sets[0]
    iters = torch.empty(B, dtype=torch.int32, device=dev)
    bp.birkhoff_fwd_ex(st["H"], st["T"], st["dual"], iters, w.tol, w.max_iter, stream)
    run_sk(st)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    hist = {int(k): int(v) for k, v in zip(*__import__("numpy").unique(it, return_counts=True))}
    waves = it[: (B // 64) * 64].reshape(-1, 64)

    def score(X):
        Xd = X.double()
        r = (Xd.sum(2) - 1).abs()
        c = (Xd.sum(1) - 1).abs()
        l1 = r.sum(1) + c.sum(1)
        resid = torch.maximum(r.amax(1), c.amax(1))
        return {"max_residual": resid.max().item(), "l1_median": l1.median().item(), "l1_max": l1.max().item()}

    b = W.bytes_per_projection(n, w.io, "fwd") * B
    digest = hipbuild.kernel_source_digest()
    return {
        "metric": "Birkhoff projections/sec (fwd only, fp32, %dx%d) on 1 MI355X" % (n, n),
        "value": B / (ms * 1e-3), "unit": "projections/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (w.key, w.title), "B": B, "n": n, "storage": w.io, "passes": "fwd",
                   "tol": w.tol, "max_iter": w.max_iter},
        "roofline": roofline(w.key, "birkhoff_fwd", b, ms, digest),
        "copy_ref": copy_reference(b, b / (ms * 1e-3) / 1e9, dev),
        "newton": dict(score(st["T"]), iterations_hist=hist, iterations_mean=float(it[it >= 0].mean()),
                       wave_max_mean=float(waves.max(1).mean()), unconverged=int((it < 0).sum())),
        "sinkhorn20": dict(score(st["S"]), ms_per_launch=ms_sk, value=B / (ms_sk * 1e-3)),
        "clock": clock,
        "kernel_digest": digest,
    }


def pages_shape_report(args, dev):
    """The pages' timing shape (Table 3 of the mHC projection paper, section 5):
    4x4 fp32 logits ~ N(0, 10^2) at B in {512, ..., 131072}.  For each B, the
    median over `--steps` single calls of the Newton forward, forward then
    backward, the one-launch forward + backward and the 20-sweep Sinkhorn-Knopp
    forward, each call timed alone with HIP events after the caches are flushed by
    writing 1 GiB; plus the accuracy of the two forwards in float64 (max
    residual and the L1 marginal error)."""
    import statistics

    import torch

    import birkhoff_projection_amd as bp
    from birkhoff_projection_amd import workloads as W

    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    rows = []
    for B in W.PAGES_SHAPE_BATCHES:
        w = W.pages_shape_workload(B)
        H = torch.from_numpy(W.make_logits(w)).to(dev)
        G = torch.from_numpy(W.make_upstream(w)).to(dev)
        T, S, dH = torch.empty_like(H), torch.empty_like(H), torch.empty_like(H)
        dual = torch.empty((B, 4), dtype=torch.float32, device=dev)
        calls = {
            "newton_fwd": lambda: bp.birkhoff_fwd(H, T, dual, w.tol, w.max_iter, stream),
            "newton_fwd_then_bwd": lambda: (bp.birkhoff_fwd(H, T, dual, w.tol, w.max_iter, stream),
                                            bp.birkhoff_bwd(H, dual, G, dH, stream)),
            "newton_fwd_bwd_one_launch": lambda: bp.birkhoff_fwd_bwd(H, G, T, dual, dH, w.tol, w.max_iter, stream),
            "sinkhorn20_fwd": lambda: bp.sinkhorn_fwd(H, S, 20, stream),
        }
        row = {"B": B}
        for name, fn in calls.items():
            for _ in range(5):
                fn()
            times = []
            for _ in range(args.steps):
                flush.fill_(1.0)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3)
            row[name + "_us"] = statistics.median(times)
        iters = torch.empty(B, dtype=torch.int32, device=dev)
        bp.birkhoff_fwd_ex(H, T, dual, iters, w.tol, w.max_iter, stream)
        bp.sinkhorn_fwd(H, S, 20, stream)
        torch.cuda.synchronize()
        for name, X in (("newton", T), ("sinkhorn20", S)):
            Xd = X.double()
            r = (Xd.sum(2) - 1).abs()
            c = (Xd.sum(1) - 1).abs()
            l1 = r.sum(1) + c.sum(1)
            row[name + "_max_residual"] = torch.maximum(r.amax(1), c.amax(1)).max().item()
            row[name + "_l1_median"] = l1.median().item()
            row[name + "_l1_max"] = l1.max().item()
        it = iters.cpu()
        row["newton_iterations_mean"] = float(it[it >= 0].float().mean())
        row["newton_unconverged"] = int((it < 0).sum())
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
    del flush
    last = rows[-1]
    return {
        "metric": "median us per call, 4x4 fp32, H~N(0,10^2), cold caches (the pages' timing shape)",
        "value": last["newton_fwd_then_bwd_us"], "unit": "us at B=%d (fwd then bwd)" % last["B"],
        "n_gpus": 1, "steps": args.steps, "warmup": 5, "higher_is_better": False, "scaling": "none",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "pages_shape: 4x4 fp32, H~N(0,10^2), dT~N(0,1), B in %s, tol 1e-6, "
                               "max_iter 100" % (list(W.PAGES_SHAPE_BATCHES),)},
        "rows": rows,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300, help="untimed steps after the settle phase")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="milliseconds of untimed back-to-back steps before the counted warm-up: the engine "
                         "clock needs tens of milliseconds of load to settle after idle")
    ap.add_argument("--workload", default="train", help="workload key (train is the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--path", choices=("fused", "separate"), default="fused",
                    help="the timed step: one birkhoff_fwd_bwd launch (fused) or birkhoff_fwd then "
                         "birkhoff_bwd (separate); the other is measured and reported alongside")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run 5 torch copies of MIB MiB (fp32) so that a counter "
                         "run can scale FETCH_SIZE / WRITE_SIZE against a copy of known size")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the projections are independent per matrix, so a "
              "multi-GPU run is the same kernel on B/N matrices per GPU with no exchange; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch

    import birkhoff_projection_amd as bp
    from birkhoff_projection_amd import workloads as W

    known = sorted(W.WORKLOADS) + sorted(W.EOT_WORKLOADS) + sorted(W.MIX_WORKLOADS) + ["pages_shape"]
    if args.workload not in known:
        print("unknown workload %r (have %s)" % (args.workload, known), file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bp.load_library()
    if args.workload == "pages_shape":
        print(json.dumps(pages_shape_report(args, dev)), flush=True)
        return 0
    if args.workload in W.EOT_WORKLOADS:
        w = W.EOT_WORKLOADS[args.workload]
        out = eot_report(w, args, dev)
    elif args.workload in W.MIX_WORKLOADS:
        w = W.MIX_WORKLOADS[args.workload]
        out = mix_report(w, args, dev)
    else:
        w = W.WORKLOADS[args.workload]
        out = forward_only_report(w, args, dev) if w.passes == "fwd" else forward_backward_report(w, args, dev)
    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": src.numel() * 4}
        del src, dst
    if not args.no_cpu_baseline:
        if args.workload in W.EOT_WORKLOADS:
            out["cpu_baseline"] = eot_cpu_baseline(w, args.cpu_seconds)
        elif args.workload in W.MIX_WORKLOADS:
            out["cpu_baseline"] = mix_cpu_baseline(w, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def copy_reference(nbytes: float, achieved_gbs: float, dev, K: int = 50) -> dict:
    """A device copy that moves the dominant kernel's algorithmic bytes per launch
    (nbytes / 2 read, nbytes / 2 written), timed like the kernels: K back-to-back
    copies alternating two buffer pairs, between two HIP events on the current
    stream.  `kernel_frac` is the kernel's achieved rate over the copy's."""
    import torch
    half = int(nbytes) // 2
    pairs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev))
             for _ in range(2)]
    for src, _ in pairs:
        src.fill_(1)
    stream = torch.cuda.current_stream(dev)
    for i in range(10):
        pairs[i % 2][1].copy_(pairs[i % 2][0])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        pairs[i % 2][1].copy_(pairs[i % 2][0])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    gbs = 2 * half / (ms * 1e-3) / 1e9
    del pairs
    torch.cuda.empty_cache()
    return {"what": "torch copy_ of %d bytes (read + write = the kernel's bytes per launch)" % half,
            "GBs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS, "kernel_frac": achieved_gbs / gbs}


def graph_replay(step, sets, K, dev):
    """ms per step when the steps are captured into a HIP graph (torch.cuda.CUDAGraph,
    50 steps per graph) and replayed: the same kernels without the host's per-launch
    work between them, as a caller that captures its step would run them.  `step`
    must launch on the current stream."""
    import torch

    per = min(K, 50)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(3):
            step(sets[i % 2])
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per):
            step(sets[i % 2])
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, K // per)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * per)
    del g
    return ms

def forward_backward_report(w, args, dev):
    """The forward + backward workloads: the timed step is the fused launch or
    the two separate launches (--path); the other form is timed too."""
    import torch

    import birkhoff_projection_amd as bp
    from birkhoff_projection_amd import build as hipbuild
    from birkhoff_projection_amd import workloads as W

    B, n = w.B, w.n
    Hs = W.make_logits(w)
    Gs = W.make_upstream(w)

    def to_dev(a):
        t = torch.from_numpy(a).to(dev)
        return t.view(torch.bfloat16) if w.io == "bf16" else t

    sets = []
    for _ in range(2):
        H = to_dev(Hs)
        G = to_dev(Gs)
        sets.append(dict(H=H, G=G, T=torch.empty_like(H), dH=torch.empty_like(H),
                         dual=torch.empty((B, n), dtype=torch.float32, device=dev)))
    del Hs, Gs
    torch.cuda.synchronize()

    fwd = bp.birkhoff_fwd if w.io == "f32" else bp.birkhoff_fwd_bf16
    bwd = bp.birkhoff_bwd if w.io == "f32" else bp.birkhoff_bwd_bf16
    fused = bp.birkhoff_fwd_bwd if w.io == "f32" else bp.birkhoff_fwd_bwd_bf16
    stream = torch.cuda.current_stream(dev)

    def run_fwd(s):
        fwd(s["H"], s["T"], s["dual"], w.tol, w.max_iter, stream)

    def run_bwd(s):
        bwd(s["H"], s["dual"], s["G"], s["dH"], stream)

    def run_fused(s):
        fused(s["H"], s["G"], s["T"], s["dual"], s["dH"], w.tol, w.max_iter, stream)

    def step_separate(s):
        run_fwd(s)
        run_bwd(s)

    step = run_fused if args.path == "fused" else step_separate

    def timed(fn, K, probe=None):
        return timed_steps(fn, sets, K, stream, probe)

    def kernel_time(fn, name):
        return per_kernel_time(fn, sets, args.steps, stream, args.settle_ms, probe, clock["mhz_after_per_kernel"], name)

    settle_steps = settle(step, sets, args.settle_ms)
    probe = bp.ClockProbe(dev)
    for i in range(args.warmup):
        step(sets[i % 2])
    torch.cuda.synchronize()

    K = args.steps
    ms_step = timed(step, K, probe)      # the timed region: K whole steps
    clock = clock_report(settle_steps, args.settle_ms, probe)
    other = step_separate if args.path == "fused" else run_fused
    ms_other = kernel_time(other, "other_path")   # the other form of the step, for comparison
    fwd_ms = kernel_time(run_fwd, "birkhoff_fwd")  # per-kernel launch times, same stream
    bwd_ms = kernel_time(run_bwd, "birkhoff_bwd")
    fused_ms = ms_step if args.path == "fused" else ms_other
    bwd_t_ms = None
    if w.io == "f32":                    # the backward from T alone (what autograd uses for fp32)
        bwd_t_ms = kernel_time(lambda s: bp.birkhoff_bwd_from_T(s["T"], s["G"], s["dH"], stream),
                               "birkhoff_bwd_from_T")

    def step_on_current(s):   # the same step, launched on whatever stream is current
        if args.path == "fused":
            fused(s["H"], s["G"], s["T"], s["dual"], s["dH"], w.tol, w.max_iter)
        else:
            fwd(s["H"], s["T"], s["dual"], w.tol, w.max_iter)
            bwd(s["H"], s["dual"], s["G"], s["dH"])

    ms_graph = graph_replay(step_on_current, sets, K, dev)

    b_fwd = W.bytes_per_projection(n, w.io, "fwd") * B
    b_bwd = W.bytes_per_projection(n, w.io, "bwd") * B
    b_fused = W.bytes_per_projection(n, w.io, "fused") * B
    if args.path == "fused":
        kern = {"birkhoff_fwd_bwd": (fused_ms, b_fused)}
    else:
        kern = {"birkhoff_fwd": (fwd_ms, b_fwd), "birkhoff_bwd": (bwd_ms, b_bwd)}
    dom = max(kern, key=lambda k: kern[k][0])
    d_ms, d_bytes = kern[dom]
    step_bytes = b_fused if args.path == "fused" else b_fwd + b_bwd
    digest = hipbuild.kernel_source_digest()

    out = {
        "metric": METRIC if (n == 4 and w.io == "f32") else
                  "%dx%d Birkhoff projections/sec (fwd+bwd, %s storage, fp32 compute) on 1 MI355X; %% HBM roofline"
                  % (n, n, w.io),
        "value": B / (ms_step * 1e-3),
        "unit": "projections/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (w.key, w.title), "B": B, "n": n, "storage": w.io,
                   "passes": "fwd+bwd", "path": args.path, "tol": w.tol, "max_iter": w.max_iter},
        "roofline": roofline(w.key, dom, d_bytes, d_ms, digest),
        "copy_ref": copy_reference(d_bytes, d_bytes / (d_ms * 1e-3) / 1e9, dev),
        "kernels_ms": dict({"birkhoff_fwd_bwd": fused_ms, "birkhoff_fwd": fwd_ms, "birkhoff_bwd": bwd_ms},
                           **({"birkhoff_bwd_from_T": bwd_t_ms} if bwd_t_ms is not None else {})),
        "step_hbm": {"algorithmic_bytes": step_bytes,
                     "achieved_GBs": step_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "other_path": {"path": "separate" if args.path == "fused" else "fused", "ms_per_step": ms_other,
                       "value": B / (ms_other * 1e-3)},
        "graph_replay": {"path": args.path, "ms_per_step": ms_graph, "value": B / (ms_graph * 1e-3)},
        "clock": clock,
        "kernel_digest": digest,
    }
    return out


if __name__ == "__main__":
    sys.exit(main())
