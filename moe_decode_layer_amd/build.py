"""Build the native parts in-tree.

* ``synth/_synth.so``  -- the seeded input generator (gcc, OpenMP).
* ``_moe_decode.so``   -- the HIP library behind the C ABI (hipcc, gfx950).

Every call compiles from source; nothing is cached.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SYNTH_SRC = os.path.join(PKG, "synth", "synth.c")
SYNTH_LIB = os.path.join(PKG, "synth", "_synth.so")
HIP_SRCS = [os.path.join(PKG, "csrc", "moe_decode.hip")]
HIP_LIB = os.path.join(PKG, "_moe_decode.so")

# Packed fp32 instructions are kept out of every device build.  The device
# compiler's atomic optimizer is off: it rewrites a one-lane fetch-add into a
# wave-wide form that waits for the result right away, which would stall the
# kernel's prefetched work claims.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_synth() -> str:
    tmp = SYNTH_LIB + ".tmp"
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, SYNTH_SRC, "-lm"])
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def build_hip() -> str:
    tmp = HIP_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-o", tmp, *HIP_SRCS])
    os.replace(tmp, HIP_LIB)
    return HIP_LIB


def build_all() -> None:
    build_synth()
    build_hip()


if __name__ == "__main__":
    what = sys.argv[1:] or ["all"]
    for w in what:
        {"synth": build_synth, "hip": build_hip, "all": build_all}[w]()
