"""Builds liblinformer.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m efficient_transformer_attention_seq_amd.build
The library lands next to this file; the binding loads it from there.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblinformer.so")

HIP_SOURCES = ["proj_bf16.hip", "attend_bf16.hip", "fused_bf16.hip", "f32_path.hip",
               "dense_bf16.hip", "linear_bf16.hip", "conv_bf16.hip", "backward_f32.hip"]
HOST_SOURCES = ["api.cpp"]  # host-only code, compiled as HIP for the runtime headers

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build liblinformer)")


def common_flags() -> list:
    return ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
            "-Wno-unused-function"]


def device_flags() -> list:
    # Packed fp32 VALU forms are disabled: hipcc would otherwise form v_pk_* fp32 ops from
    # ordinary float code.  The host pass warns that it does not know the feature (harmless).
    return ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-fno-gpu-rdc"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link liblinformer.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([cc] + common_flags() + device_flags() + ["-c", os.path.join(CSRC, src),
                                                               "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([cc] + common_flags() + device_flags() + ["-c", os.path.join(CSRC, src),
                                                               "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
