#!/usr/bin/env python3
"""rocprofv3 runs of a bench.py workload and their summary under profiles/.

    python profile_summary.py run NAME --out DIR [--bench-args "..."] [--steps K]
    python profile_summary.py summarize NAME --out DIR [--bench-args "..."]

`run` profiles `python -u bench.py <bench-args>` with rocprofv3, one pass
per counter group, each a child process under its own time limit, stopping
at the first pass that fails: a kernel trace with statistics, FETCH_SIZE,
WRITE_SIZE, three groups of other counters, and FETCH_SIZE / WRITE_SIZE of
a plain 1 GiB device copy (bench.py --copy-calibration), which scales the
two traffic counters to bytes.  Raw output stays in DIR.  `summarize` (run
by `run` at the end) writes profiles/NAME.md (commands, kernel trace table,
HBM bytes per launch against the algorithmic bytes, other counters) and
profiles/NAME_counters.json (the scaled traffic per kernel, keyed by the
digest of the device code it was taken on, which bench.py reports as
roofline.traffic while the code is unchanged).

MemUnitBusy has no gfx950 definition in rocprofv3; it is computed here from
the raw counters with the formula rocprofv3 gives for earlier gfx9 parts:
100 * max over TA units of TA_TA_BUSY / GRBM_GUI_ACTIVE of one XCD (the raw
GRBM_GUI_ACTIVE arrives summed over the XCDs).

This script never touches the GPU itself: the profiled programs run as its
child processes.
"""
import argparse
import collections
import csv
import glob
import json
import os
import shlex
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (pure Python at import: no torch, no GPU)

# counter groups of their own rocprofv3 pass each (within the per-block
# limits of one pass: at most 8 SQ, 4 TCC, 4 TCP, 2 TA, 2 GRBM counters)
GROUPS = [
    ("busy", ["TA_BUSY_max", "TA_BUSY_avr", "GRBM_GUI_ACTIVE"]),
    ("valu", ["VALUBusy", "OccupancyPercent", "MemUnitStalled"]),
    ("l2", ["TCC_HIT_sum", "TCC_MISS_sum", "SQ_LDS_BANK_CONFLICT"]),
]
COPY_BYTES = 1 << 30


def short(name):
    """rocprofv3 kernel name -> the short form bench.py and the tables use."""
    n = name.replace("void ", "", 1) if name.startswith("void ") else name
    if n.startswith("hswd::"):
        i = n.find("(hswd::")
        if i > 0:
            return n[:i] + "(...)"
    return n[:80]


def rocprof_cmd(kind, arg, out, prefix, bench_args, include=None):
    base = ["rocprofv3"]
    if kind == "trace":
        base += ["--kernel-trace", "--stats"]
    else:
        base += ["--pmc"] + arg
        if include:                  # counters of the matching kernels only
            base += ["--kernel-include-regex", include]
    return base + ["-d", out, "-o", prefix, "--output-format", "csv", "--",
                   sys.executable, "-u", "bench.py"] + bench_args


def passes(out, bench_args, steps):
    """(label, command, time limit s) of every rocprofv3 pass, in order."""
    run_args = bench_args + ["--no-cpu-baseline", "--no-ceiling", "--no-graph"]
    p = [("trace", rocprof_cmd("trace", None, os.path.join(out, "trace"), "bench",
                               run_args + ["--steps", str(steps)]), 300)]
    short_args = run_args + ["--steps", "2", "--warmup", "1"]
    for label, ctr in [("fetch", ["FETCH_SIZE"]), ("write", ["WRITE_SIZE"])] + GROUPS:
        p.append((label, rocprof_cmd("pmc", ctr, os.path.join(out, label), "bench", short_args,
                                     "hswd"), 240))
    for label, ctr in [("copyf", ["FETCH_SIZE"]), ("copyw", ["WRITE_SIZE"])]:
        p.append((label, rocprof_cmd("pmc", ctr, os.path.join(out, label), "copy",
                                     ["--copy-calibration"], "copy"), 120))
    return p


def run(args):
    os.makedirs(args.out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for label, cmd, limit in passes(args.out, shlex.split(args.bench_args), args.steps):
        print("profile pass %s: %s" % (label, " ".join(cmd)), flush=True)
        with open(os.path.join(args.out, label + ".log"), "w") as log:
            r = subprocess.run(["timeout", "-s", "KILL", str(limit)] + cmd, cwd=ROOT, env=env,
                               stdout=log, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            # rocprofv3 itself may end with a segmentation fault after the
            # program finished and its results are whole: accept that only
            # when the program's own last line made it out
            tail = open(os.path.join(args.out, label + ".log")).read().splitlines()[-3:]
            done = any(t.startswith("{") or "copy calibration" in t for t in tail)
            if not (r.returncode == 139 and done):
                print("profile pass %s failed with status %d" % (label, r.returncode), flush=True)
                return r.returncode
        print("profile pass %s done" % label, flush=True)
    rc = summarize(args)
    if rc == 0 and args.prune:
        # the raw per-dispatch tables are large (torch's kernel names run to
        # kilobytes); the statistics and agent tables stay
        for f in glob.glob(os.path.join(args.out, "**", "*.csv"), recursive=True):
            if f.endswith(("_kernel_trace.csv", "_counter_collection.csv")):
                os.remove(f)
    return rc


def _csv(out, label, kind):
    files = glob.glob(os.path.join(out, label, "**", "*_%s.csv" % kind), recursive=True)
    if not files:
        raise FileNotFoundError("no %s csv under %s/%s" % (kind, out, label))
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def counter_means(out, label):
    """{short kernel name: {counter: mean per dispatch}, with dispatch counts}."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv(out, label, "counter_collection"):
        acc[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in d.items()} for k, d in acc.items()}


def gpu_xcds(out, label):
    """XCD count of the profiled GPU (rocprofv3's agent information)."""
    for r in _csv(out, label, "agent_info"):
        if r["Agent_Type"] == "GPU":
            return int(r["Num_Xcc"])
    raise ValueError("no GPU agent in %s/%s" % (out, label))


def copy_value(out, label, counter):
    vals = [float(r["Counter_Value"]) for r in _csv(out, label, "counter_collection")
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
    return max(vals)


def algorithmic_bytes(bench_args):
    """{short kernel name: algorithmic bytes per launch} for the workload."""
    a = argparse.ArgumentParser()
    a.add_argument("--workload", default="step28_64x4096_bf16")
    a.add_argument("--kv", default="bf16")
    a.add_argument("--heads", type=int, default=bench.H)
    ns, _ = a.parse_known_args(bench_args)
    if ns.workload != "step28_64x4096_bf16":
        kind, B_, dtype, pos, seed, Hq = bench.SINGLE_LAYER[ns.workload][:6]
        g, pieces = (bench.kernel_group("fp8" if dtype == "fp8" else "bf16", Hq)
                     if Hq > bench.HKV else (1, 1))
        code = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}[dtype]
        name = "hswd::attn_kernel<256, %d, %s, 1, %d, %s>(...)" % (
            code, "true" if kind == "sliding" else "false", g, "true" if pieces > 1 else "false")
        return {name: bench.single_layer_bytes(ns.workload)}
    elt = 1 if ns.kv == "fp8" else 2
    full = bench.full_kernel(ns.kv, ns.heads)
    return {full: bench.layer_bytes("full", elt=elt, heads=ns.heads),
            full.replace(", false, 1,", ", true, 1,", 1): bench.layer_bytes("sliding", elt=elt,
                                                                           heads=ns.heads)}


def summarize(args):
    out = args.out
    bench_args = shlex.split(args.bench_args)
    alg = algorithmic_bytes(bench_args)
    lines = ["# %s" % args.name, "",
             "Device: AMD Instinct MI355X (gfx950), ROCm 7.2, one GPU.", "",
             "Made by `python profile_summary.py run %s --out <dir> --bench-args %s --steps %d` "
             "from the repository root, which runs these passes (each a rocprofv3 process of "
             "its own):" % (args.name, shlex.quote(args.bench_args), args.steps), ""]
    for label, cmd, _ in passes("<dir>", bench_args, args.steps):
        lines.append("    " + " ".join(shlex.quote(c) if c != sys.executable else "python"
                                       for c in cmd))
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    stats = sorted(_csv(out, "trace", "kernel_stats"), key=lambda r: -float(r["Percentage"]))
    for r in stats[:8]:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    avg_us = {short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}

    cf = copy_value(out, "copyf", "FETCH_SIZE")
    cw = copy_value(out, "copyw", "WRITE_SIZE")
    fs, ws = COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw
    fetch = counter_means(out, "fetch")
    write = counter_means(out, "write")
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              "Scale: a plain 1 GiB device copy reads FETCH_SIZE = %.1f KiB and WRITE_SIZE = %.1f "
              "KiB for 1048576 KiB moved each way, so FETCH_SIZE x %.4f and WRITE_SIZE x %.4f are "
              "bytes (KiB x 1024)." % (cf, cw, fs, ws), "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB | "
              "algorithmic MB | HBM / algorithmic | avg us | GB/s (algorithmic) | % of 8 TB/s |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    record = {"code_digest": bench.kernel_source_digest(),
              "digest_of": "device code: csrc/kernels/*.hpp, csrc/attn_launch.hpp, "
                           "csrc/attn_g*.hip",
              "fetch_scale": fs, "write_scale": ws, "bench_args": args.bench_args,
              "kernels": {}}
    for k in sorted(fetch):
        if not k.startswith("hswd::"):
            continue
        fv, n = fetch[k]["FETCH_SIZE"]
        wv = write.get(k, {}).get("WRITE_SIZE", (0.0, 0))[0]
        rb, wb = fv * 1024 * fs, wv * 1024 * ws
        a = alg.get(k)
        us = avg_us.get(k)
        lines.append("| %s | %d | %.1f | %.1f | %.2f | %.2f | %s | %s | %s | %s | %s |" % (
            k, n, fv, wv, rb / 1e6, wb / 1e6, "%.2f" % (a / 1e6) if a else "-",
            "%.4f" % ((rb + wb) / a) if a else "-", "%.1f" % us if us else "-",
            "%.0f" % (a / (us * 1e-6) / 1e9) if a and us else "-",
            "%.1f" % (a / (us * 1e-6) / 1e9 / bench.PEAK_HBM_GBS * 100) if a and us else "-"))
        record["kernels"][k] = {"read_bytes": rb, "write_bytes": wb, "fetch_kib": fv,
                                "write_kib": wv, "dispatches": n, "avg_us": us,
                                "algorithmic_bytes": a}

    lines += ["", "## Other counters (one rocprofv3 --pmc pass per group)", "",
              "| kernel | counter | mean per dispatch | pass (--pmc ...) |", "|---|---|---|---|"]
    derived = []
    for label, ctrs in GROUPS:
        try:
            means = counter_means(out, label)
        except FileNotFoundError:
            derived.append("(counter pass %s: %s not collected)" % (label, " ".join(ctrs)))
            continue
        for k in sorted(means):
            if not k.startswith("hswd::attn"):
                continue
            for c in ctrs:
                if c in means[k]:
                    lines.append("| %s | %s | %.2f | %s |" % (k, c, means[k][c][0], " ".join(ctrs)))
            if label == "busy" and "TA_BUSY_max" in means[k] and "GRBM_GUI_ACTIVE" in means[k]:
                # GRBM_GUI_ACTIVE comes summed over the XCDs; every XCD runs
                # the kernel for its whole duration, so one XCD's count is
                # the sum over the XCD count
                xcd = gpu_xcds(out, label)
                active = means[k]["GRBM_GUI_ACTIVE"][0] / xcd
                mub = 100 * means[k]["TA_BUSY_max"][0] / active
                mua = 100 * means[k]["TA_BUSY_avr"][0] / active
                derived.append("MemUnitBusy of %s: %.1f%% (busiest TA unit; %.1f%% on average "
                               "over TA units; GRBM_GUI_ACTIVE %.0f cycles per XCD)."
                               % (k, mub, mua, active))
                record["kernels"].setdefault(k, {})["mem_unit_busy"] = mub
            if label == "l2" and "TCC_HIT_sum" in means[k] and "TCC_MISS_sum" in means[k]:
                h, m = means[k]["TCC_HIT_sum"][0], means[k]["TCC_MISS_sum"][0]
                derived.append("L2 hit rate of %s: %.2f%%." % (k, 100 * h / max(h + m, 1)))
    lines += [""] + derived + ["",
              "MemUnitBusy = 100 x TA_BUSY_max / GRBM_GUI_ACTIVE of one XCD (rocprofv3 "
              "defines no MemUnitBusy for gfx950; this is its formula for earlier gfx9 parts, "
              "whose GRBM_GUI_ACTIVE is taken as a maximum over instances; here the raw counter "
              "arrives summed over the 8 XCDs and is divided by their count). The kernel "
              "trace covers every launch of its run (parity pass, warmup and timed steps) and "
              "torch's seeded data generation and copies (at::native kernels, copyBuffer), which "
              "are set-up, not the decode path. Algorithmic bytes: valid K/V rows plus per-stream "
              "inputs and outputs (bench.py layer_bytes / single_layer_bytes)."]
    for d in [os.path.join(ROOT, "profiles")] + ([args.copy_to] if args.copy_to else []):
        os.makedirs(d, exist_ok=True)
        md = os.path.join(d, args.name + ".md")
        with open(md, "w") as f:
            f.write("\n".join(lines) + "\n")
        with open(os.path.join(d, args.name + "_counters.json"), "w") as f:
            json.dump(record, f, indent=1)
        print("wrote %s" % md, flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("action", choices=["run", "summarize"])
    ap.add_argument("name")
    ap.add_argument("--out", required=True)
    ap.add_argument("--bench-args", default="")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--copy-to", default=None,
                    help="also write the summary files into this directory")
    ap.add_argument("--no-prune", dest="prune", action="store_false",
                    help="keep the raw per-dispatch csv tables after summarising")
    args = ap.parse_args()
    sys.exit(run(args) if args.action == "run" else summarize(args))


if __name__ == "__main__":
    main()
