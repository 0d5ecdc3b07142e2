"""Build libpa.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Run ``python -m paged_kv_cache_267_amd.build`` (or ``__graft_entry__.build()``).
Every source is compiled on each call; objects go to ``_build/``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libpa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 instructions stay off (see the device code notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LDS is laid out by the kernels themselves: per-thread arrays stay in
    # registers instead of being moved into spare LDS by the compiler
    "-mllvm", "-disable-promote-alloca-to-lds",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
