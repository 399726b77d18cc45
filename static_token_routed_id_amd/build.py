"""Build libl3.so for gfx950 (MI355X) with hipcc, in-tree.

Usage: python -m static_token_routed_id_amd.build [--jobs N]

Every HIP source under csrc/ and the C-ABI layer are compiled to objects
under _build/ and linked into static_token_routed_id_amd/libl3.so. The build
runs on any machine with ROCm (hipcc cross-compiles gfx950 code without a GPU).
csrc/read_probe.hip, a read-bandwidth probe that bench.py times beside the
gather, goes into libl3probe.so of its own.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libl3.so")
# read-bandwidth probe, a library of its own (measurement only)
PROBE_LIB = os.path.join(PKG, "libl3probe.so")
ARCH = os.environ.get("L3_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are switched off for every device compile.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]

SOURCES = ["plan.hip", "seg_fwd.hip", "seg_group.hip", "gemm.hip", "bwd.hip",
           "stage.hip",
           "api.cpp", "alloc.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmds.append([HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src),
                                              "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp]
         + objs)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC] + FLAGS + ["-shared", "-x", "hip",
                            os.path.join(CSRC, "read_probe.hip"), "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    sys.exit(0)
