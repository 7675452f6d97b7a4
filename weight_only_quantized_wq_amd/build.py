"""Build libwq.so (HIP, gfx950) in-tree next to this file.

    python -m weight_only_quantized_wq_amd.build      # or build() from Python

Compiles every ``csrc/*.hip`` with hipcc for gfx950 into one shared library.
Packed fp32 VALU instructions are disabled for the device code
(``-target-feature -packed-fp32-ops``); the host pass ignores that flag with
a warning.
"""

import glob
import os
import shutil
import subprocess
import sys

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


def command(out=LIB, extra=()):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        *extra, *sources(), "-o", out,
    ]


def build(verbose=False):
    """Compile libwq.so; raises CalledProcessError on a compile error."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
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
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
