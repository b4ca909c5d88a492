"""Compile libmoba.so for gfx950 in-tree: one hipcc job per source, then a link.

    python block_sparse_long_pool_amd/build.py [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoba.so")
SOURCES = ["pool.hip", "gate.hip", "index.hip", "attn.hip", "attn_bwd.hip", "conv.hip",
           "decode.hip", "moba_api.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 ops stay off: only ordinary fp32 instructions are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")
    return r


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_host_asan(out_dir: str | None = None, jobs: int | None = None) -> str:
    """The same library with its HOST code built with AddressSanitizer (the device code
    is unchanged): libmoba_asan.so, for the CPU tests of the argument checks and the
    workspace arithmetic.  Load it in a process that preloads the clang ASan runtime
    (asan_runtime())."""
    out_dir = out_dir or os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        _run([HIPCC, *COMMON, *san, "-c", os.path.join(CSRC, src), "-o", obj], False)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(out_dir, "libmoba_asan.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
          "-fsanitize=address", "-o", lib, *objs], False)
    return lib


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that matches hipcc's host compiler."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
