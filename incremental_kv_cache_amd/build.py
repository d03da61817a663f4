"""Builds libkvcache.so in-tree: HIP kernels for gfx950 plus the host cache manager.

    python -m incremental_kv_cache_amd.build

The kernels are compiled with hipcc for gfx950 only.  Packed-FP32 instruction
selection is switched off for all device code (``-target-feature
-packed-fp32-ops``); hipcc's host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvcache.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]

DEVICE_SOURCES = ["kvc_device.hip", "kvc_decode.hip", "kvc_mfma.hip", "kvc_probe.hip"]
HOST_SOURCES = ["kvc_host.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compiles every HIP source for gfx950 and links libkvcache.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run(["g++", *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
