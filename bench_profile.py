#!/usr/bin/env python3
"""Summarise rocprofv3 output of bench.py runs into profiles/ (text only).

    # kernel durations: rocprofv3 --kernel-trace --stats --output-format csv \
    #     -d OUT -o bench -- python bench.py [bench args]
    python bench_profile.py trace OUT/bench_kernel_stats.csv OUT/bench_kernel_trace.csv \
        --bench-log BENCH.log --cmd "<the rocprofv3 command>" --out profiles/NAME.md

    # HBM traffic: two counter runs (FETCH_SIZE, then WRITE_SIZE) of the same
    # bench command; the 1 GiB device copy bench.py issues before timing
    # (__amd_rocclr_copyBuffer) calibrates both counters
    python bench_profile.py traffic FETCH.csv WRITE.csv --sha SOURCE_SHA \
        --class "int4g32 m=1 k=4096=gemv_kernel<wq::FmtInt4, 1, 2, 2, 4, false>" \
        --cmd "<fetch command>" --cmd "<write command>" --out profiles/NAME.md

    # other counters (SQ_* instruction mix), one csv per pass
    python bench_profile.py pmc PASS1.csv PASS2.csv --sha SOURCE_SHA --cmd ... --out profiles/NAME.md

The traffic summary also merges its classes into profiles/traffic.json,
which bench.py reads for the roofline's `traffic` field while the kernel
sources still hash to SOURCE_SHA.
"""

import argparse
import collections
import csv
import json
import os
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def _short(name):
    return name.split("(")[0].replace("void ", "")


def _per_matrix(rows, workload, steps):
    """Per-matrix durations of a `--launch per-matrix` run: the first `steps`
    steps' dispatches of the step kernels come in the workload's matrix order
    (warmup and eager steps), so dispatch i is matrix i mod the step's count."""
    import sys
    sys.path.insert(0, ROOT)
    from synth.workloads import WORKLOADS
    from weight_only_quantized_wq_amd.layerset import matrix_bytes
    wl = WORKLOADS[workload]
    mats = wl.matrices()
    ks = [r for r in rows if "wq::" in r["Kernel_Name"] and "quantize" not in r["Kernel_Name"]]
    ks.sort(key=lambda r: int(r["Start_Timestamp"]))
    ks = ks[:steps * len(mats)]
    per = collections.defaultdict(list)
    kern = {}
    for i, r in enumerate(ks):
        m = mats[i % len(mats)]
        key = (m.name, m.n, m.k)
        per[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        kern[key] = _short(r["Kernel_Name"])
    lines = ["", f"## Per matrix (first {steps} steps of `{workload}`, one launch per matrix, in matrix order)", "",
             "| matrix | n x k | kernel | launches | median us | GB/s (algorithmic) | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for (name, n, k), v in per.items():
        med = statistics.median(v)
        b = matrix_bytes(wl.fmt, n, k, wl.m)
        lines.append(f"| {name} | {n} x {k} | `{kern[(name, n, k)]}` | {len(v)} | {med / 1e3:.2f} | "
                     f"{b / med:.0f} | {b / med / 8000 * 100:.1f} |")
    return lines


def trace(args):
    stats = list(csv.DictReader(open(args.stats)))
    rows = list(csv.DictReader(open(args.trace)))
    per = collections.defaultdict(list)
    for r in rows:
        if "wq::" not in r["Kernel_Name"]:
            continue
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        per[(_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))].append(d)
    lines = ["# rocprofv3 kernel trace: " + args.title, "", f"Kernel sources: `{args.sha}` (bench.py `source_sha`).",
             "", "Command (run from /tmp, repository root in $R):", "",
             "    " + args.cmd, "", "## Kernel stats (libwq kernels; all dispatches of the run)", "",
             "| kernel | calls | average ns | min ns | max ns | share of GPU time |", "|---|---|---|---|---|---|"]
    for s in stats:
        if "wq::" in s["Name"]:
            lines.append(f"| `{_short(s['Name'])}` | {s['Calls']} | {float(s['AverageNs']):.0f} | {s['MinNs']} | "
                         f"{s['MaxNs']} | {float(s['Percentage']):.1f}% |")
    lines += ["", "## Per launch shape (workgroups per launch)", "",
              "| kernel | workgroups | dispatches | mean us | median us |", "|---|---|---|---|---|"]
    for (k, wg), v in sorted(per.items()):
        lines.append(f"| `{k}` | {wg} | {len(v)} | {statistics.mean(v) / 1e3:.2f} | {statistics.median(v) / 1e3:.2f} |")
    if args.per_matrix:
        wl, steps = args.per_matrix.split(":")
        lines += _per_matrix(rows, wl, int(steps))
    if args.bench_log:
        bl = [l.rstrip() for l in open(args.bench_log) if l.startswith("[bench]")]
        lines += ["", "## bench.py lines of the profiled run", ""] + ["    " + l for l in bl]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print(args.out)


def _counter(path, cname):
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == cname:
            out[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def traffic(args):
    f = _counter(args.fetch, "FETCH_SIZE")
    w = _counter(args.write, "WRITE_SIZE")
    # the calibration copy is the largest device copy of the run (a workload
    # may copy smaller buffers while it is built)
    copy_f = max(f["__amd_rocclr_copyBuffer"]) * 1024
    copy_w = max(w["__amd_rocclr_copyBuffer"]) * 1024
    sf, sw = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    table = {}
    lines = ["# rocprofv3 HBM traffic: " + args.title, "", "Commands (run from /tmp, repository root in $R):", ""]
    lines += ["    " + c for c in args.cmd]
    lines += ["", f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {copy_f / 1024:.0f} KiB and "
              f"WRITE_SIZE = {copy_w / 1024:.0f} KiB, so fetch counts are scaled by {sf:.4f} and write counts "
              f"by {sw:.4f}.", "", "| class | kernel | dispatches | fetch bytes/launch | write bytes/launch | "
              "total bytes/launch |", "|---|---|---|---|---|---|"]
    for spec in args.klass:
        cls, kern = spec.rsplit("=", 1)
        fv = [v for k, vv in f.items() if k.endswith(kern) for v in vv]
        wv = [v for k, vv in w.items() if k.endswith(kern) for v in vv]
        fb = statistics.mean(fv) * 1024 * sf
        wb = statistics.mean(wv) * 1024 * sw
        table[cls] = {"kernel": kern, "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
                      "bytes_per_launch": int(fb + wb), "dispatches": len(fv)}
        lines.append(f"| {cls} | `{kern}` | {len(fv)} | {fb:.0f} | {wb:.0f} | {fb + wb:.0f} |")
    lines = lines[:2] + [f"Kernel sources: `{args.sha}` (bench.py `source_sha`).", ""] + lines[2:]
    open(args.out, "w").write("\n".join(lines) + "\n")
    # merge into profiles/traffic.json (entries of other sources are dropped)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        doc = json.load(open(path))
    except (OSError, ValueError):
        doc = {}
    if doc.get("source_sha") != args.sha:
        doc = {"source_sha": args.sha, "kernels": {}, "summaries": []}
    for cls, e in table.items():
        e["fetch_scale"], e["write_scale"] = sf, sw
        e["summary"] = os.path.relpath(args.out, ROOT)
        doc["kernels"][cls] = e
    doc.setdefault("summaries", [])
    if os.path.relpath(args.out, ROOT) not in doc["summaries"]:
        doc["summaries"].append(os.path.relpath(args.out, ROOT))
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
    print(args.out)


def pmc(args):
    """Per-kernel means of arbitrary counters (one or more counter csv files)."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in args.csv:
        for r in csv.DictReader(open(path)):
            if "wq::" not in r["Kernel_Name"] or "quantize" in r["Kernel_Name"]:
                continue
            key = f"{_short(r['Kernel_Name'])} ({int(r['Grid_Size']) // int(r['Workgroup_Size'])} workgroups)"
            agg[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in agg for c in agg[k]})
    lines = ["# rocprofv3 counters: " + args.title, "", f"Kernel sources: `{args.sha}` (bench.py `source_sha`).", "",
             "Commands (run from /tmp, repository root in $R):", ""] + ["    " + c for c in args.cmd] + [
             "", "Mean per dispatch (counters summed over the device).", "",
             "| kernel | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for k in sorted(agg):
        n = max(len(v) for v in agg[k].values())
        lines.append(f"| `{k}` | {n} | " + " | ".join(f"{statistics.mean(agg[k][c]):.4g}" if agg[k].get(c) else ""
                                                   for c in names) + " |")
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print(args.out)


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("trace")
    t.add_argument("--bench-log")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="bench.py")
    t.add_argument("--sha", default="")
    t.add_argument("--per-matrix", help="WORKLOAD:STEPS -- per-matrix table of a --launch per-matrix run")
    t.add_argument("--out", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch")
    c.add_argument("write")
    c.add_argument("--sha", required=True)
    c.add_argument("--class", dest="klass", action="append", required=True)
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--title", default="bench.py")
    c.add_argument("--out", required=True)
    q = sub.add_parser("pmc")
    q.add_argument("csv", nargs="+")
    q.add_argument("--sha", required=True)
    q.add_argument("--cmd", action="append", required=True)
    q.add_argument("--title", default="bench.py")
    q.add_argument("--note", default="")
    q.add_argument("--out", required=True)
    a = p.parse_args()
    {"trace": trace, "traffic": traffic, "pmc": pmc}[a.what](a)


if __name__ == "__main__":
    main()
