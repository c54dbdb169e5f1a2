"""Build libmoe.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m mixture_experts_transformer_sigmoid_amd.build [--sanitize]

Always recompiles every source; objects go to _build/, the library next to this file.
--sanitize builds _build/san/libmoe_san.so instead: the host side under AddressSanitizer
and UndefinedBehaviorSanitizer, for the host-side tests.
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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build: every source compiled with
# the sanitizers on its host pass only (each -fsanitize right after -Xarch_host; the device
# code is the normal gfx950 build), linked against the shared sanitizer runtime.  Loaded
# by a process that preloads that runtime (see sanitizer_env).
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libmoe_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The shared ASan runtime of the ROCm clang that built the library."""
    out = _run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"]).strip().splitlines()[-1]
    if not os.path.exists(out):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("ASan runtime not found")
        out = hits[0]
    return out


def build_sanitized(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(SAN_DIR, exist_ok=True)
    objs, jobs = [], []
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1"] + SAN_FLAGS
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 8)) as ex:
        for src in SOURCES:
            obj = os.path.join(SAN_DIR, src.replace(".hip", ".o"))
            objs.append(obj)
            jobs.append(ex.submit(_run, [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", "-Xarch_host",
          "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", SAN_LIB, *objs])
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def sanitizer_env() -> dict:
    """Environment for a child process that loads the sanitized library through the
    binding: the ASan runtime preloaded (the Python interpreter is not instrumented), leak
    checks off (the interpreter's own allocations), every report fatal."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["MOE_LIB"] = SAN_LIB
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sanitize":
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
