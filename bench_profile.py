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

The traffic summary also writes profiles/traffic.json, which bench.py reads
for the roofline's `traffic` field while the kernel sources still hash to
SOURCE_SHA.
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


def trace(args):
    stats = list(csv.DictReader(open(args.stats)))
    rows = list(csv.DictReader(open(args.trace)))
    per = collections.defaultdict(list)
    for r in rows:
        if "wq::" not in r["Kernel_Name"]:
            continue
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        per[(_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))].append(d)
    lines = ["# rocprofv3 kernel trace: " + args.title, "", "Command (run from /tmp, repository root in $R):", "",
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
    copy_f = statistics.mean(f["__amd_rocclr_copyBuffer"]) * 1024
    copy_w = statistics.mean(w["__amd_rocclr_copyBuffer"]) * 1024
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
    open(args.out, "w").write("\n".join(lines) + "\n")
    doc = {"source_sha": args.sha, "fetch_scale": sf, "write_scale": sw, "kernels": table,
           "summary": os.path.relpath(args.out, ROOT)}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
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
    t.add_argument("--out", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch")
    c.add_argument("write")
    c.add_argument("--sha", required=True)
    c.add_argument("--class", dest="klass", action="append", required=True)
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--title", default="bench.py")
    c.add_argument("--out", required=True)
    a = p.parse_args()
    trace(a) if a.what == "trace" else traffic(a)


if __name__ == "__main__":
    main()
