"""Condense rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m birkhoff_projection_amd.profile_summary --workload train \\
        --stats prof/kt_train --fetch prof/pmc_fetch --write prof/pmc_write \\
        --copy-mib 512 --cmd-stats "..." --cmd-fetch "..." --cmd-write "..." [--sq prof/pmc_sq --cmd-sq "..."]

Inputs are the directories rocprofv3 wrote with `--output-format csv`:
  --stats  a `--kernel-trace --stats` run (reads *_kernel_stats.csv);
  --fetch  a `--pmc FETCH_SIZE` run, --write a `--pmc WRITE_SIZE` run (reads
           *_counter_collection.csv); both runs also executed a device copy of
           --copy-mib MiB (bench.py --calibrate-copy), whose counter readings
           give the factor that turns each counter into bytes;
  --sq     optionally, a run of SQ_* / GRBM_* counters (raw sums per dispatch).

Writes profiles/kernels_<workload>.md, profiles/traffic_<workload>.md and
profiles/traffic_<workload>.json (bytes per launch, read by bench.py together
with the digest of the kernel sources the counters were taken on).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import pathlib
import statistics

from . import build as hipbuild

ROOT = pathlib.Path(__file__).resolve().parent.parent

# device kernel -> the C-ABI entry point that launches it
ENTRY = (("newton_fwd_kernel", "birkhoff_fwd"), ("newton_fwd_gather_kernel", "birkhoff_fwd"),
         ("implicit_bwd_from_T_kernel", "birkhoff_bwd_from_T"),
         ("implicit_bwd_kernel", "birkhoff_bwd"),
         ("sinkhorn_kernel", "sinkhorn_fwd"), ("fused_fwd_bwd_kernel", "birkhoff_fwd_bwd"),
         ("eot_fwd_kernel", "birkhoff_eot_fwd"), ("eot_bwd_kernel", "birkhoff_eot_bwd"),
         ("project_mix_kernel", "birkhoff_fwd_mix"), ("mix_bwd_kernel", "birkhoff_mix_bwd"))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def entry_of(kernel_name: str):
    for key, entry in ENTRY:
        if key in kernel_name:
            return entry
    return None


def stats_variant(kernel_name: str) -> bool:
    """The forward kernels' variant that also writes iteration counts (template flag true)."""
    return ("fwd_kernel<" in kernel_name or "fwd_gather_kernel<" in kernel_name) and "true>" in kernel_name


def one_csv(d: pathlib.Path, suffix: str) -> pathlib.Path:
    found = sorted(pathlib.Path(d).rglob("*" + suffix))
    if not found:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return found[0]


def kernel_stats(d):
    rows = list(csv.DictReader(open(one_csv(d, "_kernel_stats.csv"))))
    return [{"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
             "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
             "pct": float(r["Percentage"])} for r in rows]


def loop_averages(d, last=0):
    """Average duration (us) of each kernel over its longest run of consecutive
    dispatches -- the back-to-back launches bench.py times with events -- or
    over the final `last` dispatches of that run (the timed ones, when the run
    also holds the warm-up launches)."""
    rows = list(csv.DictReader(open(one_csv(d, "_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    best = {}
    run_name, run = None, []
    for r in rows + [None]:
        name = r["Kernel_Name"] if r else None
        if name != run_name:
            if run_name is not None and len(run) > len(best.get(run_name, [])):
                best[run_name] = run
            run_name, run = name, []
        if r:
            run.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if last > 0:
        best = {k: v[-last:] for k, v in best.items()}
    return {k: (len(v), sum(v) / len(v)) for k, v in best.items()}


def counters(d):
    """{(kernel name, counter): [value per dispatch]}"""
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(one_csv(d, "_counter_collection.csv"))):
        out[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return out


def last_copy(d, counter):
    """The counter's reading for the run's last device copy: bench.py's
    calibration copies come after all timed work, so the last copy dispatch is
    one of them (uploads of inputs earlier in the run may have any size)."""
    best = None
    for r in csv.DictReader(open(one_csv(d, "_counter_collection.csv"))):
        if COPY_KERNEL in r["Kernel_Name"] and r["Counter_Name"] == counter:
            k = int(r["Dispatch_Id"])
            if best is None or k > best[0]:
                best = (k, float(r["Counter_Value"]))
    return None if best is None else best[1]


def per_kernel(cnt, counter):
    return {k: statistics.median(v) for (k, c), v in cnt.items() if c == counter}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--stats", required=True, action="append",
                    help="a kernel-trace directory; may be repeated (one section each)")
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--cmd-stats", required=True, action="append")
    ap.add_argument("--cmd-fetch", required=True)
    ap.add_argument("--cmd-write", required=True)
    ap.add_argument("--sq")
    ap.add_argument("--cmd-sq")
    ap.add_argument("--bench-json", action="append", default=[],
                    help="bench.py JSON line of each traced run, in the order of --stats")
    ap.add_argument("--timed", type=int, default=0,
                    help="bench.py --steps of the traced runs: average only the last this many launches "
                         "of each back-to-back run")
    ap.add_argument("--out", default=str(ROOT / "profiles"))
    a = ap.parse_args()
    out = pathlib.Path(a.out)
    out.mkdir(parents=True, exist_ok=True)
    digest = hipbuild.kernel_source_digest()

    if len(a.cmd_stats) != len(a.stats):
        raise SystemExit("give one --cmd-stats per --stats")
    lines = ["# Kernel durations, workload `%s`" % a.workload, "",
             "Kernel sources digest `%s`. Durations are rocprofv3 kernel-trace times per dispatch "
             "(warm-up launches included). Commands run from /tmp with TMPDIR=/tmp; `$R` is the "
             "repository root." % digest]
    for k_run, (d, cmd) in enumerate(zip(a.stats, a.cmd_stats)):
        lines += ["", "## Run %d" % (k_run + 1), "", "    " + cmd, "",
                  "| kernel | entry point | calls | avg us | min us | max us | % of GPU time |",
                  "|---|---|---|---|---|---|---|"]
        for r in kernel_stats(d):
            lines.append("| `%s` | %s | %d | %.2f | %.2f | %.2f | %.1f |" % (
                r["name"].split("(")[0], entry_of(r["name"]) or "-", r["calls"], r["avg_us"], r["min_us"],
                r["max_us"], r["pct"]))
        la = loop_averages(d, a.timed)
        lines += ["", "Back-to-back launches of one kernel alone (the longest run of consecutive dispatches "
                  "of each kernel%s; bench.py times the same loops with HIP events):" % (
                      ", its last %d launches" % a.timed if a.timed else ""), "",
                  "| kernel | entry point | launches | avg us |", "|---|---|---|---|"]
        for k, (cnt, avg) in sorted(la.items()):
            lines.append("| `%s` | %s | %d | %.2f |" % (k.split("(")[0], entry_of(k) or "-", cnt, avg))
        if k_run < len(a.bench_json):
            b = json.loads(pathlib.Path(a.bench_json[k_run]).read_text().strip().splitlines()[-1])
            per = b.get("kernels_ms")
            if per is None:   # forward-only report: the forward and the Sinkhorn baseline
                per = {"birkhoff_fwd": b["ms_per_step"]}
                if "sinkhorn20" in b:
                    per["sinkhorn_fwd"] = b["sinkhorn20"]["ms_per_launch"]
            lines += ["", "bench.py's own HIP-event figures in the same run (path `%s`): %s ms per step; "
                      "per-kernel average launch %s ms." % (
                          b["config"].get("path", "separate"), round(b["ms_per_step"], 5),
                          {k: round(v, 5) for k, v in per.items()})]
    (out / ("kernels_%s.md" % a.workload)).write_text("\n".join(lines) + "\n")

    fc, wc = counters(a.fetch), counters(a.write)
    f_k, w_k = per_kernel(fc, "FETCH_SIZE"), per_kernel(wc, "WRITE_SIZE")
    copy_bytes = a.copy_mib << 20
    f_copy = [last_copy(a.fetch, "FETCH_SIZE")]
    w_copy = [last_copy(a.write, "WRITE_SIZE")]
    if f_copy[0] is None or w_copy[0] is None:
        raise SystemExit("the counter runs hold no %s dispatch to calibrate against" % COPY_KERNEL)
    f_scale = copy_bytes / f_copy[0]     # bytes per FETCH_SIZE unit
    w_scale = copy_bytes / w_copy[0]     # bytes per WRITE_SIZE unit
    traffic = {}
    rows = []
    for k in sorted(set(f_k) | set(w_k)):
        e = entry_of(k)
        if e is None:
            continue
        rd = f_k.get(k, float("nan")) * f_scale
        wr = w_k.get(k, float("nan")) * w_scale
        if not stats_variant(k):   # the timed launches are the ones without iteration counts
            traffic[e] = rd + wr
        rows.append("| `%s` | %s | %.0f | %.0f | %.1f | %.1f | %.1f |" % (
            k.split("(")[0], e, f_k.get(k, float("nan")), w_k.get(k, float("nan")), rd / 1e6, wr / 1e6,
            (rd + wr) / 1e6))
    doc = ["# HBM traffic per launch, workload `%s`" % a.workload, "",
           "Commands (run from /tmp with TMPDIR=/tmp; `$R` is the repository root):", "",
           "    " + a.cmd_fetch, "    " + a.cmd_write, "",
           "FETCH_SIZE and WRITE_SIZE are in KiB per dispatch as rocprofv3 reports them. The same runs copy "
           "%d MiB five times at their end with a device copy kernel (`%s`); the last copy's readings "
           "(FETCH %.0f, WRITE %.0f) give "
           "the factors that turn the counters into bytes: %.4f bytes per FETCH unit and %.4f per WRITE unit "
           "(a counter that counted KiB exactly would give 1024)." % (
               a.copy_mib, COPY_KERNEL, f_copy[0], w_copy[0], f_scale, w_scale), "",
           "Kernel sources digest `%s` (bench.py uses these figures only while the digest matches)." % digest,
           "",
           "| kernel | entry point | FETCH_SIZE | WRITE_SIZE | read MB | written MB | traffic MB |",
           "|---|---|---|---|---|---|---|"] + rows
    if a.sq:
        sq = counters(a.sq)
        names = sorted({c for (_, c) in sq})
        doc += ["", "## SQ / GRBM counters (sum over the chip, median per dispatch)", "",
                "    " + (a.cmd_sq or ""), "",
                "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
        kern = sorted({k for (k, _) in sq if entry_of(k)})
        for k in kern:
            doc.append("| `%s` | " % k.split("(")[0] + " | ".join(
                "%.4g" % statistics.median(sq[(k, c)]) if (k, c) in sq else "-" for c in names) + " |")
    valu, active = {}, {}
    if a.sq:
        for (k, c), v in counters(a.sq).items():
            e = entry_of(k)
            if e is None or stats_variant(k):
                continue
            if c == "SQ_INSTS_VALU":
                valu[e] = statistics.median(v)
            elif c == "SQ_ACTIVE_INST_VALU":
                active[e] = statistics.median(v)
    (out / ("traffic_%s.md" % a.workload)).write_text("\n".join(doc) + "\n")
    (out / ("traffic_%s.json" % a.workload)).write_text(json.dumps(
        {"workload": a.workload, "kernel_digest": digest, "bytes_per_launch": traffic,
         "valu_insts_per_launch": valu, "valu_active_per_launch": active,
         "fetch_scale": f_scale, "write_scale": w_scale}, indent=1) + "\n")
    print("\n".join(lines + [""] + doc))


if __name__ == "__main__":
    main()
