"""Build the gfx950 shared library ``libmoe_mi355x.so`` from ``csrc/``.

Every translation unit is compiled by hipcc for gfx950 only, in parallel, and
linked into one shared library in this package directory (in-tree, so it
travels with the source tree). Packed-fp32 instructions are disabled for all
device code.

Usage: ``python -m sparsely_gated_mixture_moe_amd.build [--jobs N] [--incremental]``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "moe_mi355x")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h")))


def _compile(src: str, incremental: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(p) for p in [src] + headers())
        if os.path.getmtime(obj) >= newest:
            return obj
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + DEVICE_FLAGS + lang + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(jobs: int = 0, incremental: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--incremental", action="store_true")
    a = ap.parse_args()
    build(a.jobs, a.incremental)
