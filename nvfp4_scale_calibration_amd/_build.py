"""Build liblh.so (the HIP/gfx950 C-ABI library) in-tree with hipcc.

Flags: gfx950 only; -O3; IEEE fp32 (no fast-math, FP contraction off, so
every fma in the kernels is written explicitly); packed-fp32 instruction
selection disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblh.so")
SOURCES = ["lh_api.hip", "lh_hessian.hip", "lh_sweep.hip", "lh_quant.hip", "lh_dense.hip"]
HEADERS = ["lh_device.h", "lh_internal.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def build(force: bool = True, verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every source in parallel, then link liblh.so.  Returns its path."""
    if not force and os.path.exists(LIB):
        return LIB
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    objs, failed = [], []
    for src, obj, p in procs:
        out, _ = p.communicate()
        if verbose or p.returncode != 0 or resource_usage:
            sys.stderr.write(out)
        if p.returncode != 0:
            failed.append(src)
        objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(force=True, verbose="-v" in sys.argv, resource_usage="--usage" in sys.argv)
    print(LIB)
