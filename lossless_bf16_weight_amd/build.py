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


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    dev_o = os.path.join(BUILD, "uw_device.o")
    host_o = os.path.join(BUILD, "uw_host.o")
    jobs = [
        [hipcc] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-c", os.path.join(CSRC, "uw_device.hip"), "-o", dev_o],
        ["g++"] + CXX_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-c", os.path.join(CSRC, "uw_host.cpp"), "-o", host_o],
    ]
    with ThreadPoolExecutor(2) as ex:
        outs = list(ex.map(run, jobs))
    tmp = LIB + ".tmp"
    outs.append(run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, dev_o, host_o, "-o", tmp, "-lpthread"]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.verbose))
    sys.exit(0)
