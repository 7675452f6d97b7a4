"""Build libwq.so (HIP, gfx950) in-tree next to this file.

    python -m weight_only_quantized_wq_amd.build      # or build() from Python

Compiles every ``csrc/*.hip`` with hipcc for gfx950 (one object per source,
compiled in parallel) and links them into one shared library.  Packed fp32
VALU instructions are disabled for the device code
(``-target-feature -packed-fp32-ops``); the host pass ignores that flag with
a warning.
"""

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwq.so")
ARCH = "gfx950"


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libwq)")
    return exe


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def compile_command(src, obj, extra=()):
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(HERE, "csrc"), *extra, "-c", src, "-o", obj]


def link_command(objs, out):
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, err)
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def build(verbose=False, jobs=None):
    """Compile libwq.so; raises CalledProcessError on a compile error."""
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="wqbuild") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, compile_command(s, o), verbose) for s, o in zip(srcs, objs)]:
                f.result()
        tmp = LIB + ".tmp"
        _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
