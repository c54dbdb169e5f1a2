"""Build libmoe.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m mixture_experts_transformer_sigmoid_amd.build

Always recompiles every source; objects go to _build/, the library next to this file.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

SOURCES = ["route.hip", "permute.hip", "ffn.hip", "ffn_fp8.hip", "combine.hip", "moe_abi.hip"]

ARCH = "gfx950"
# packed fp32 instructions are switched off for all device code (they are not emitted
# by hand either); hipcc's host pass warns that it does not know the feature.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmoe)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 8)) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
