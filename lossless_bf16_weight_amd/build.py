"""Build libuw.so in-tree for gfx950: hipcc for the device code, g++ for the host codec.

    python -m lossless_bf16_weight_amd.build [--jobs N]

The library lands next to this file (lossless_bf16_weight_amd/libuw.so); intermediate
objects go to _build/ at the repository root.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libuw.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
               # packed fp32 instructions are kept out of every kernel
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
             "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]


def run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


# Device sources (each compiled on its own, in parallel) and the host codec.
HIP_SOURCES = ("uw_gemm.hip", "uw_decode.hip", "uw_glue.hip", "uw_capi.hip")
HOST_SOURCES = ("uw_host.cpp",)


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    objs, cmds = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append(["g++"] + CXX_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(jobs or min(len(cmds), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(run, cmds))
    tmp = LIB + ".tmp"
    outs.append(run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp, "-lpthread"]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--jobs", type=int, default=None, help="parallel compiles (default: one per source)")
    args = ap.parse_args()
    print(build(args.verbose, args.jobs))
    sys.exit(0)
