"""Builds libmoe_mi355x.so (HIP, gfx950) in-tree with hipcc.

    python -m mixture_experts_layer_38_amd.build [--debug]

--debug builds libmoe_mi355x_debug.so instead: the same kernels with
device-side bounds checks on every index read from memory (MOE_DEBUG).
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
# the debug build: device-side bounds checks on every index read from memory
BUILD_DEBUG = os.path.join(PKG, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libmoe_mi355x_debug.so")
SOURCES = ["moe_api.hip", "router.hip", "dispatch.hip", "grouped_gemm.hip", "grouped_gemm_f8.hip", "grouped_gemm_bwd.hip",
           "stream_gemm.hip",
           "simple_f32.hip", "balance.hip", "quant_e4m3.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
    "-Wno-unused-function", "-I", INCLUDE,
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8, debug: bool = False) -> str:
    """Compiles every HIP source for gfx950 and links the shared library
    (debug: the bounds-checked library, -DMOE_DEBUG)."""
    bdir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    flags = FLAGS + (["-DMOE_DEBUG"] if debug else [])
    os.makedirs(bdir, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for pr in procs:
        _wait(pr, verbose)
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} in {time.time() - t0:.1f}s")
    return lib


def _wait(pr, verbose):
    cmd, p = pr
    out, _ = p.communicate()
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
