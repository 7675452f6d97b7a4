"""Host logic of the benchmark and its profile summaries (CPU only).

The roofline arithmetic, the traffic lookup's source-hash check, the
counter calibration of the profile summaries, the algorithmic byte counts
per format and the workloads' matrix sets -- none of which needs a GPU.
"""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_device_warmup_is_explicit_and_can_be_switched_off():
    """The untimed device warm-up before the warmup steps is a flag of its
    own (recorded in the line), and 0 skips it without touching the GPU."""
    import bench
    assert bench.parse([]).device_warmup_ms == 60.0
    assert bench.parse(["--device-warmup-ms", "0"]).device_warmup_ms == 0.0
    assert bench.device_warmup(0) == 0


def test_roofline_takes_the_class_with_the_most_time():
    import bench
    launches = [("a", 0, 1e9), ("a", 0, 1e9), ("b", 0, 6e9)]
    dur = {"a": (0.4, [0, 1]), "b": (1.0, [2])}      # ms per launch: a 0.8 ms per step, b 1.0 ms
    dom, roof = bench.roofline(launches, dur)
    assert dom == "b"
    assert roof["achieved"] == pytest.approx(6000.0)          # 6 GB in 1 ms
    assert roof["frac"] == pytest.approx(6000.0 / bench.HBM_PEAK_GBS)
    assert roof["launches_per_step"] == 1 and roof["bound"] == "hbm"
    assert roof["avg_launch_us"] == pytest.approx(1000.0)
    assert roof["all_kernels_gbs"] == pytest.approx(8e9 / 1.8e-3 / 1e9, abs=0.1)


def test_traffic_is_reported_only_for_the_counted_sources(tmp_path, monkeypatch):
    import bench
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"source_sha": "abc", "kernels": {"k": {"bytes_per_launch": 123}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("k", "abc") == 123
    assert bench.traffic_for("k", "abd") is None
    assert bench.traffic_for("other", "abc") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("k", "abc") is None


def _counter_csv(path, name, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kern, value in rows:
            w.writerow({"Kernel_Name": kern, "Counter_Name": name, "Counter_Value": value})


def test_traffic_summary_scales_counters_by_the_copy_kernel(tmp_path, monkeypatch):
    import bench_profile
    # the 1 GiB copy reads 0.5 GiB of FETCH_SIZE (scale 2) and 1 GiB of WRITE_SIZE (scale 1), in KiB
    copy = "__amd_rocclr_copyBuffer"
    kern = "void wq::some_kernel<1>(args)"
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 524288), (kern, 1000), (kern, 1002)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1048576), (kern, 10), (kern, 10)])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench_profile, "ROOT", str(tmp_path))
    args = type("A", (), {})()
    args.fetch, args.write, args.sha = str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "s1"
    args.klass = ["cls=some_kernel<1>"]
    args.cmd, args.title, args.out = ["c1", "c2"], "t", str(tmp_path / "profiles" / "x.md")
    bench_profile.traffic(args)
    doc = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert doc["source_sha"] == "s1"
    e = doc["kernels"]["cls"]
    assert e["fetch_scale"] == pytest.approx(2.0) and e["write_scale"] == pytest.approx(1.0)
    assert e["fetch_bytes_per_launch"] == int(1001 * 1024 * 2.0)
    assert e["write_bytes_per_launch"] == 10 * 1024
    assert e["dispatches"] == 2
    # a second summary of the same sources merges; another source starts over
    args.klass, args.out = ["cls2=some_kernel<1>"], str(tmp_path / "profiles" / "y.md")
    bench_profile.traffic(args)
    doc = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert set(doc["kernels"]) == {"cls", "cls2"} and len(doc["summaries"]) == 2
    args.sha = "s2"
    bench_profile.traffic(args)
    doc = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert doc["source_sha"] == "s2" and set(doc["kernels"]) == {"cls2"}


@pytest.mark.parametrize("fmt,group", [("int4g32", 32), ("int4g64", 64), ("int4g128", 128), ("int4g256", 256),
                                       ("int4pc", None), ("int8", None), ("bf16", None)])
def test_weight_bytes_match_what_the_quantizers_write(fmt, group):
    """The bench's byte count per format equals the sizes of the arrays the
    (oracle) quantizers produce for that format."""
    from weight_only_quantized_wq_amd.layerset import weight_bytes, matrix_bytes
    from oracle.quant import quantize_int4, quantize_int8
    n, k = 3, 512
    w = np.zeros((n, k), np.float32)
    if fmt.startswith("int4"):
        p, sz = quantize_int4(w, group or k)
        want = p.nbytes + sz.nbytes
    elif fmt == "int8":
        q, s = quantize_int8(w)
        want = q.nbytes + s.nbytes
    else:
        want = 2 * n * k
    assert weight_bytes(fmt, n, k) == want
    assert matrix_bytes(fmt, n, k, m=5) == want + 2 * 5 * k + 2 * 5 * n


def test_workload_matrix_sets():
    from synth.workloads import WORKLOADS
    assert len(WORKLOADS["llama2-7b-int4"].matrices()) == 32 * 4 + 1
    assert len(WORKLOADS["llama3.1-70b-int4-m5"].matrices()) == 80 * 4 + 1
    assert WORKLOADS["llama3.1-70b-int8-m5"].matrices() == WORKLOADS["llama3.1-70b-int4-m5"].matrices()
    assert len(WORKLOADS["int8-4096"].matrices()) == 64
    shapes = {(m.n, m.k) for m in WORKLOADS["llama2-7b-int4"].matrices()}
    assert shapes == {(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008), (32000, 4096)}


def test_context_figures_are_the_pages_rows():
    """The bench line's context block repeats the pages' printed figures
    (tests/golden/pages_benchmark_rows.json, each row cited there)."""
    import bench
    rows = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_benchmark_rows.json")))["rows"]
    key = {("A100", "llama-2-7b"): "a100_llama2_7b", ("A100", "llama-2-70b"): "a100_llama2_70b",
           ("A100", "llama-3.1-8b"): "a100_llama3_1_8b", ("A100", "llama-3.1-70b"): "a100_llama3_1_70b",
           ("MI250X-GCD", "llama-2-7b"): "mi250x_gcd_llama2_7b"}
    seen = 0
    for r in rows:
        e = bench.PAGES_CONTEXT[key[(r["hw"], r["model"])]][r["format"]]
        assert e["tok_per_s"] == r["tok_s"] and e["gbs"] == r["gb_s"]
        seen += 1
    assert seen == len(rows) == 10
    assert bench.PAGES_CONTEXT["a100_mixtral_8x7b"]["int8"]["tok_per_s"] == 97.92


def test_host_threads_and_cpu_model(monkeypatch):
    import bench
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_threads() == (1, n)
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_threads() == (n, n)
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_cpu_samples_extrapolate_row_slices_to_the_step(monkeypatch):
    """A slice of rows stands for its full matrix in proportion n / rows, and
    each shape counts as often as the step holds it."""
    import bench
    from synth.configs import Model
    from synth.workloads import Workload
    from weight_only_quantized_wq_amd.layerset import matrix_bytes
    tiny = Model("tiny", 64, 96, 128, 160, 3)
    wl = Workload("tiny-int4", 99, "int4g32", 1, 0.02, tiny)
    monkeypatch.setattr(bench, "_time_repeated", lambda fn, s: (fn(), 1e-3)[1])
    rows, sample = bench.cpu_samples(wl, 0.01, max_weights=64 * 40)
    got = {shape: (count, t, b) for shape, count, t, b in rows}
    assert set(got) == {(96, 64), (64, 64), (256, 64), (64, 128), (160, 64)}
    assert got[(256, 64)] == (3, pytest.approx(1e-3 * 256 / 40), matrix_bytes("int4g32", 256, 64))
    assert got[(64, 128)] == (3, pytest.approx(1e-3 * 64 / 20), matrix_bytes("int4g32", 64, 128))
    assert got[(160, 64)][0] == 1
    assert "[40x64] of [256x64]" in sample


def test_tensor_parallel_shards_split_rows_or_inputs():
    """One GPU's shard under P-way tensor parallelism: wqkv and w1|w3 keep
    1/P of their rows, wo and w2 1/P of their inputs, lm_head stays whole."""
    from synth.workloads import WORKLOADS
    for p in (2, 4, 8):
        full = WORKLOADS["llama2-7b-int4"].matrices()
        shard = WORKLOADS[f"llama2-7b-int4-tp{p}"].matrices()
        assert len(full) == len(shard)
        for a, b in zip(full, shard):
            if a.name in ("wqkv", "w13"):
                assert (b.n, b.k) == (a.n // p, a.k)
            elif a.name in ("wo", "w2"):
                assert (b.n, b.k) == (a.n, a.k // p)
            else:
                assert (b.n, b.k) == (a.n, a.k)
            assert b.k % 32 == 0 and b.n * p in (a.n, a.n * p)
    s8 = {(m.n, m.k) for m in WORKLOADS["llama3.1-70b-int4-m5-tp8"].matrices()}
    assert s8 == {(1280, 8192), (8192, 1024), (7168, 8192), (8192, 3584), (128256, 8192)}
    assert WORKLOADS["llama3.1-70b-int4-m5-tp8"].m == 5
