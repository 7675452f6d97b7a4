#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s of weight-only quantized decode matvecs on MI355X.

One step = one batch-1 decode step's linear layers (all matvecs of the
workload) with inputs already resident in HBM: by default one persistent
launch (two for the MoE layers) issued directly per step; with
``--launch per-matrix`` one launch per matrix, captured once into a HIP graph
and replayed per step.
Default workload: the Llama-2-7B linear set in int4 G=32 (129 matvecs,
4.1337 GB per step).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line.  `value` is whole-step throughput in GB/s of
algorithmic bytes (weights + scales/zeros + bf16 activations in and out)
over the wall time of K steps; `roofline` reports the dominant kernel's
achieved GB/s from HIP-event durations of its launches (the events around
the K timed steps for a fused step; per-matrix launches are captured as one
graph per kernel class and replayed K times), against the 8 TB/s HBM peak;
`cpu_baseline` times the CPU oracle (fp64 dequantize + BLAS matvec) on a
bounded sample of the same workload, extrapolated to a whole step.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) + equiv. batch-1 decode tok/s, Llama-2-7B int4 G=32"
METRIC_OTHER = "achieved HBM GB/s (% of peak) + equiv. batch-1 decode tok/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # 20 warmup steps: the step kernels re-cut their workgroups' ranges from
    # the balance state each launch measures (settled within a few launches);
    # an idle device's ramp is taken by --device-warmup-ms
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama2-7b-int4")
    p.add_argument("--launch", choices=("fused", "per-matrix"), default="fused",
                   help="linear sets: one persistent launch per step (default) or one launch per matrix")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time for the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-calibration", action="store_true", help="skip the 1 GiB copy used to scale PMC counters")
    p.add_argument("--device-warmup-ms", type=float, default=60.0,
                   help="untimed HBM streaming through a scratch buffer before the warmup steps (0: none)")
    p.add_argument("--no-graph", action="store_true",
                   help="fused steps: skip the HIP-graph replay timed for comparison (kernel traces then hold "
                        "only the direct launches)")
    return p.parse_args(argv)


def source_sha():
    h = hashlib.sha256()
    base = os.path.join(ROOT, "weight_only_quantized_wq_amd", "csrc")
    for name in sorted(os.listdir(base)):
        with open(os.path.join(base, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def build_workload(name, launch="fused"):
    import torch
    from synth.workloads import WORKLOADS, gen_w_device, gen_x_device, expert_key, logits_key, moe_x_key
    from synth.gen import device_normal, device_bf16_normal
    from weight_only_quantized_wq_amd.layerset import LayerSet, MoELayerSet
    wl = WORKLOADS[name]
    if wl.fmt == "int8" and wl.model is not None and wl.model.name.startswith("mixtral"):
        mm = wl.model

        def gw(rows, cols, key):
            return device_normal((rows, cols), wl.sigma, "cuda", *expert_key(wl, key[0], key[1], key[2]))

        def gx(dim, layer):
            return device_bf16_normal((dim,), "cuda", *moe_x_key(wl, layer))

        def gl(e, layer):
            return device_normal((e,), 1.0, "cuda", *logits_key(wl, layer))
        ls = MoELayerSet(mm.dim, mm.ffn, mm.experts, mm.layers, gw, gx, gl)
        if launch == "fused":
            ls.prepare_fused()
            launches = [(f"moe step kernels int8 top-2 ({mm.layers} layers: W13 pass + W2 pass)", 0, ls.bytes)]
            return wl, ls, launches, lambda i: ls.step_fused(), ls.step_fused
        launches = [("moe_top2_gemv", mm.dim, ls.bytes / mm.layers)] * mm.layers
        return wl, ls, launches, ls.launch_layer, ls.step
    ls = LayerSet(wl.matrices(), wl.fmt, gen_w_device(wl), gen_x_device(wl), m=wl.m)
    if wl.model is None:
        # every copy holds the same seed-0 weights
        for q in ls.mats[1:]:
            q.w.copy_(ls.mats[0].w)
            q.aux.copy_(ls.mats[0].aux)
            q.x.copy_(ls.mats[0].x)
    torch.cuda.synchronize()
    if launch == "fused":
        ls.prepare_fused()
        launches = [(f"decode step kernel {wl.fmt} m={wl.m} ({len(ls.mats)} matrices)", 0, ls.bytes)]
        return wl, ls, launches, lambda i: ls.step_fused(), ls.step_fused
    launches = [(f"{wl.fmt} m={q.m} k={q.k}", q.k, q.bytes) for q in ls.mats]
    return wl, ls, launches, lambda i: ls.mats[i].launch(), ls.step


def copy_calibration():
    """A plain 1 GiB device copy: the PMC runs scale FETCH_SIZE / WRITE_SIZE by
    what these counters read for it (1 GiB read, 1 GiB written)."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def device_warmup(ms):
    """Streams a 256 MiB scratch buffer (not the workload's) through HBM for
    about `ms` milliseconds.  A device that was idle runs its first ~20
    launches up to 5 % slower; fresh plans on a warm device do not (the
    balance state plays no part), so this brings the device, not the plan,
    to its sustained state before the warmup steps."""
    import torch
    if ms <= 0:
        return 0
    src = torch.empty(1 << 26, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):
            dst.copy_(src)
        torch.cuda.synchronize()
        n += 16
    del src, dst
    return n


def capture(fn):
    """Capture fn's launches (on torch's current stream inside the capture)
    into a HIP graph; the workload has already run eagerly, so every lazily
    initialised host-side cache in the library is warm."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_steps(step, steps):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def timed_steps_events(step, steps):
    """Wall time of `steps` steps and the HIP-event span (ms) around them,
    both events recorded on torch's current stream (where the steps run)."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, a.elapsed_time(b)


def kernel_durations(launch_one, launches, steps):
    """Average duration (ms) of one launch of each launch class, from HIP events.

    A class is one kernel configuration (format, tokens per pass, K).  The
    launches of each class in one step are captured back to back into one HIP
    graph; each of `steps` replays is bracketed by a pair of events recorded
    on torch's current stream (the stream the graph runs on), and the average
    launch duration is the events' elapsed time over the number of launches.
    Events around every single launch would add their own processing time (a
    few microseconds) to each microsecond-scale kernel, and eager launches of
    small kernels are bound by the host, not the GPU.
    """
    import torch
    classes = {}
    for i, (cls, _, _) in enumerate(launches):
        classes.setdefault(cls, []).append(i)

    def runner(idx):
        def run():
            for i in idx:
                launch_one(i)
        return run
    graphs = {c: capture(runner(idx)) for c, idx in classes.items()}
    out = {}
    for c, idx in classes.items():
        g = graphs[c]
        g.replay()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / steps
        out[c] = (ms / len(idx), idx)
    del graphs
    return out


def roofline(launches, dur):
    """Dominant kernel = launch class with the most time per step; achieved =
    its algorithmic bytes per launch over its average launch duration."""
    best = None
    all_bytes = all_ms = 0.0
    for cls, (ms_per_launch, idx) in dur.items():
        nbytes = sum(launches[i][2] for i in idx)
        t_ms = ms_per_launch * len(idx)
        all_bytes += nbytes
        all_ms += t_ms
        if best is None or t_ms > best[2]:
            best = (cls, nbytes, t_ms, len(idx))
    dom, nbytes, t_ms, count = best
    achieved = nbytes / (t_ms * 1e-3) / 1e9
    return dom, {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": None,
        "kernel": dom,
        "launches_per_step": count,
        "avg_launch_us": round(t_ms / count * 1e3, 3),
        "avg_bytes_per_launch": int(nbytes / count),
        "all_kernels_gbs": round(all_bytes / (all_ms * 1e-3) / 1e9, 1),
    }


def traffic_for(dom, sha):
    """HBM bytes per launch from committed PMC summaries, if they were taken
    on the current kernel sources; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = t.get("kernels", {}).get(dom)
    if not entry or t.get("source_sha") != sha:
        return None
    return entry.get("bytes_per_launch")


# The pages' own batch-1 figures (gittoolsai "gpt-fast" README mirror, tables
# "基准测试" and "AMD"): whole-model decode tokens/s and the memory bandwidth
# they report, on other hardware.  Context for the bench line, not a target.
PAGES_CONTEXT = {
    "source": "gittoolsai 'gpt-fast' README mirror, tables '基准测试' (A100-80GB at 330 W, batch 1) and 'AMD' "
              "(one MI250X GCD); whole-model tokens/s on other hardware, context only",
    "a100_llama2_7b": {"bf16": {"tok_per_s": 104.9, "gbs": 1397.31}, "int8": {"tok_per_s": 155.58, "gbs": 1069.20},
                       "int4g32": {"tok_per_s": 196.80, "gbs": 862.69}},
    "a100_llama2_70b": {"int8": {"tok_per_s": 19.13, "gbs": 1322.58}, "int4g32": {"tok_per_s": 25.25, "gbs": 1097.66}},
    "a100_llama3_1_8b": {"bf16": {"tok_per_s": 93.89, "gbs": 1410.76}, "int8": {"tok_per_s": 137.64, "gbs": 1030.89}},
    "a100_llama3_1_70b": {"int8": {"tok_per_s": 18.04, "gbs": 1253.78}},
    "a100_mixtral_8x7b": {"int8": {"tok_per_s": 97.92}},
    "mi250x_gcd_llama2_7b": {"bf16": {"tok_per_s": 76.33, "gbs": 1028.70}, "int8": {"tok_per_s": 101.86, "gbs": 700.06}},
}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo ("unknown" if unreadable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """CPUs this process may run on, capped by OMP_NUM_THREADS when it is set
    (the box's share of the host for one GPU)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return (min(n, cap) if cap > 0 else n), n


def _time_repeated(fn, seconds):
    """Calls fn until `seconds` have passed (at least twice); seconds per call."""
    fn()
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 >= seconds and reps >= 2:
            break
    return (time.perf_counter() - t0) / reps


def cpu_samples(wl, budget_s, max_weights=1 << 22):
    """The oracle (fp64 dequantize + BLAS matvec) on one row slice of each
    distinct matrix shape of the workload, host-generated and quantized by
    the oracle (not timed).  Returns (rows of (shape, count in the step,
    seconds per call of the full matrix, algorithmic bytes of the full
    matrix), sample text).  A slice holds at most `max_weights` weights; the
    oracle's work is linear in the rows, so a full matrix costs n / rows
    slices."""
    import numpy as np
    from oracle.quant import quantize_int8, quantize_int4
    from oracle.bf16 import round_f32_to_bf16
    from oracle.matvec import gemv_bf16, gemv_int8, gemv_int4, gemm_small_m, gemm_small_m_int8
    from oracle.moe import expert_ffn
    from synth.gen import host_normal, host_bf16_normal
    from weight_only_quantized_wq_amd.layerset import matrix_bytes, moe_layer_bytes, int4_group
    out = []
    if wl.model is not None and wl.model.name.startswith("mixtral"):
        # one expert's SwiGLU FFN at a quarter of the ffn width, scaled by 4
        # (its work is linear in f); a layer runs two experts
        mm = wl.model
        d, f = mm.dim, mm.ffn // 4
        q13, s13 = quantize_int8(host_normal((2 * f, d), 0.02, 77, 0, 0))
        q2, s2 = quantize_int8(host_normal((d, f), 0.02, 77, 0, 1))
        x = host_bf16_normal((d,), 77, 9)
        t = _time_repeated(lambda: expert_ffn(x, q13, s13, q2, s2), budget_s)
        out.append(((2 * mm.ffn, d), mm.layers, 2 * 4 * t, moe_layer_bytes(d, mm.ffn)))
        return out, f"one int8 expert FFN [{2 * f}x{d}] + [{d}x{f}] (a quarter of the ffn width), x4 for the " \
                    f"full expert, x2 experts per layer, x{mm.layers} layers"
    shapes = {}
    for mat in wl.matrices():
        shapes.setdefault((mat.n, mat.k), [mat, 0])[1] += 1
    per = budget_s / max(1, len(shapes))
    parts = []
    for (n, k), (mat, count) in shapes.items():
        rows = max(1, min(n, max_weights // max(k, 1)))
        w = host_normal((rows, k), wl.sigma, 78, mat.mid, k)
        x = host_bf16_normal((wl.m, k) if wl.m > 1 else (k,), 78, mat.mid, 1)
        g = int4_group(wl.fmt, k)
        if g:
            p, sz = quantize_int4(w, g)
            fn = (lambda x=x, p=p, sz=sz: gemm_small_m(x, p, sz)) if wl.m > 1 else \
                 (lambda x=x, p=p, sz=sz: gemv_int4(x, p, sz))
        elif wl.fmt == "int8":
            q, sc = quantize_int8(w)
            fn = (lambda x=x, q=q, sc=sc: gemm_small_m_int8(x, q, sc)) if wl.m > 1 else \
                 (lambda x=x, q=q, sc=sc: gemv_int8(x, q, sc))
        else:
            wb = round_f32_to_bf16(w)
            fn = lambda x=x, wb=wb: gemv_bf16(x, wb)
        t = _time_repeated(fn, per)
        out.append(((n, k), count, t * n / rows, matrix_bytes(wl.fmt, n, k, wl.m)))
        parts.append(f"[{rows}x{k}] of [{n}x{k}] (x{count})")
    return out, "row slices " + ", ".join(parts) + ", each scaled to its full matrix and summed over the step"


def cpu_baseline(wl_name, target_s):
    """The CPU oracle timed on the host's cores on a bounded sample of the
    workload, extrapolated to one whole step (stated in `sample`); plus the
    single int8 GEMV 4096 x 4096 on one core."""
    from threadpoolctl import threadpool_limits, threadpool_info
    from synth.workloads import WORKLOADS
    from oracle.quant import quantize_int8
    from oracle.matvec import gemv_int8
    from synth.workloads import host_int8_4096
    wl = WORKLOADS[wl_name]
    threads, affinity = host_threads()
    with threadpool_limits(limits=threads, user_api="blas"):
        used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        rows, sample = cpu_samples(wl, target_s)
    step_s = sum(count * t for _, count, t, _ in rows)
    step_bytes = sum(count * b for _, count, _, b in rows)
    # the single int8 GEMV (4096 x 4096, seed 0) on one core
    w, x = host_int8_4096()
    q, sc = quantize_int8(w)
    with threadpool_limits(limits=1, user_api="blas"):
        t1 = _time_repeated(lambda: gemv_int8(x, q, sc), 2.0)
    from weight_only_quantized_wq_amd.layerset import matrix_bytes
    return {"value": round(step_bytes / step_s / 1e9, 3), "unit": "GB/s", "cores": int(used), "kind": "oracle",
            "sample": f"{sample} (fp64 dequantize single-threaded numpy, matvec BLAS with {used} threads); "
                      f"extrapolated step {step_s:.3f} s",
            "step_s_extrapolated": round(step_s, 4), "affinity_cpus": affinity, "cpu_model": cpu_model(),
            "int8_gemv_4096_one_core_gbs": round(matrix_bytes("int8", 4096, 4096) / t1 / 1e9, 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not a benchmark.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    t_build = time.perf_counter()
    wl, ls, launches, launch_one, step = build_workload(args.workload, args.launch)
    from weight_only_quantized_wq_amd.layerset import MoELayerSet
    print(f"[bench] built {args.workload}: {len(launches)} launches, {ls.bytes / 1e9:.4f} GB/step "
          f"in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)
    if not args.no_calibration:
        copy_calibration()
    device_warmup(args.device_warmup_ms)

    fused = hasattr(ls, "plan")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timing = {}
    if fused:
        # a fused step is one launch (two for the MoE layers): issued
        # directly, back to back on torch's current stream, bracketed by HIP
        # events on that stream; the events' span over K steps is the step
        # kernel's average duration (consecutive launches leave no gap)
        wall, ev_ms = timed_steps_events(step, args.steps)
        dur = {launches[0][0]: (ev_ms / args.steps / len(launches), list(range(len(launches))))}
        if not args.no_graph:
            # the same step replayed from a HIP graph, for comparison only
            graph = capture(step)
            for _ in range(args.warmup):
                graph.replay()
            g_wall = timed_steps(graph.replay, args.steps)
            timing["graph_replay_ms_per_step"] = round(g_wall / args.steps * 1e3, 4)
            print(f"[bench] same step replayed from a HIP graph: {g_wall / args.steps * 1e3:.3f} ms/step",
                  file=sys.stderr, flush=True)
            del graph
    else:
        eager = timed_steps(step, args.steps)
        timing["eager_ms_per_step"] = round(eager / args.steps * 1e3, 4)
        print(f"[bench] eager launches: {eager / args.steps * 1e3:.3f} ms/step", file=sys.stderr, flush=True)
        graph = capture(step)
        for _ in range(args.warmup):
            graph.replay()
        wall = timed_steps(graph.replay, args.steps)
        dur = None
    ms_per_step = wall / args.steps * 1e3
    gbs = ls.bytes * args.steps / wall / 1e9
    print(f"[bench] timed {args.steps} steps ({'direct launches' if fused else 'graph replays'}): "
          f"{ms_per_step:.3f} ms/step, {gbs:.1f} GB/s", file=sys.stderr, flush=True)

    if dur is None:
        dur = kernel_durations(launch_one, launches, args.steps)
    dom, roof = roofline(launches, dur)
    sha = source_sha()
    roof["traffic"] = traffic_for(dom, sha)
    print(f"[bench] dominant kernel {dom}: {roof['achieved']} GB/s per launch ({roof['frac'] * 100:.1f}% of peak)",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_seconds)
        print(f"[bench] cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC if wl.name == "llama2-7b-int4" else f"{METRIC_OTHER}, {wl.name}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "device_warmup_ms": args.device_warmup_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tok_per_s_equiv": round(1e3 / ms_per_step, 1),
        "tok_per_s_equiv_note": ("linear layers only; an upper bound for a decode step, whose layers depend on "
                                 "each other" + (" (here fused into one launch)" if hasattr(ls, "plan") else "")),
        "config": {
            "workload": wl.name,
            "weights": wl.fmt,
            "tokens_per_pass": wl.m,
            "launches_per_step": len(launches),
            "copies_per_step": len(ls.mats) if wl.model is None else None,
            "bytes_per_step": int(ls.bytes),
            "batch": 1,
            "launch": ((("two persistent launches per step (all layers' W13, then all layers' W2)"
                         if isinstance(ls, MoELayerSet) else "one persistent launch per step")
                        + ", issued directly") if fused else "one launch per matrix, replayed from a HIP graph"),
        },
        "timing": timing,
        "roofline": roof,
        "cpu_baseline": cpu,
        "context": PAGES_CONTEXT,
        "source_sha": sha,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
