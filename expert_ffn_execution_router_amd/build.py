"""Builds libmoe.so (HIP kernels for gfx950 + host C++) in the package directory.

The host FFN path is compiled with g++ for the host ISA (x86-64-v3: AVX2 and
FMA); the kernels and the C ABI are compiled with hipcc for gfx950 only.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

HIP_SOURCES = ["route.hip", "gemm_dec.hip", "gemm_pf.hip", "gemv.hip", "gemm_pf8.hip", "combine.hip", "slots.hip",
               "noalloc.hip"]
# Per-source code-generation options (none at present).
HIP_EXTRA = {}
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + CSRC, "-I" + os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).splitlines()
    noise = "is not a recognized feature for this target"
    msgs = [l for l in out if noise not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd[:3]))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    procs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(["hipcc", *HIP_FLAGS, *HIP_EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    api_obj = os.path.join(BUILD, "api.o")
    objs.append(api_obj)
    procs.append(["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj])
    host_obj = os.path.join(BUILD, "host_ffn.o")
    objs.append(host_obj)
    procs.append(["g++", "-O3", "-march=x86-64-v3", "-std=c++20", "-fPIC", "-Wall", "-pthread",
                  "-I" + CSRC, "-c", os.path.join(CSRC, "host_ffn.cpp"), "-o", host_obj])
    # compile in parallel
    running = []
    for cmd in procs:
        running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = False
    for cmd, p in running:
        out, err = p.communicate()
        noise = "is not a recognized feature for this target"
        msgs = [l for l in (out + err).splitlines() if noise not in l]
        if msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
        if p.returncode != 0:
            failed = True
    if failed:
        raise RuntimeError("compilation failed")
    tmp = LIB + ".tmp"
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
