"""Build libpagedattn.so in-tree for gfx950.

    python -m paged_variable_length_amd.build        # or build() from Python

Host C++ (task table, packing, validation) is compiled with g++; the HIP kernels and launchers
with hipcc for gfx950; both are linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedattn.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    """Compile every source and link LIB; returns its path. Always rebuilds."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    host_o = os.path.join(out_dir, "host.o")
    _run(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-c",
          os.path.join(CSRC, "host.cpp"), "-o", host_o] + inc)
    dev_objs = []
    for name in ("attention", "gemm"):
        obj = os.path.join(out_dir, name + ".o")
        # packed-fp32 instructions are disabled for all device code
        _run([_hipcc(), f"--offload-arch={ARCH}", "-std=c++17", "-O3", "-fPIC", "-c",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              os.path.join(CSRC, name + ".hip"), "-o", obj] + inc)
        dev_objs.append(obj)
    tmp = LIB + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", host_o] + dev_objs +
         ["-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
