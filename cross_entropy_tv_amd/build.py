"""Build the HIP library in-tree for gfx950.

    python cross_entropy_tv_amd/build.py

compiles csrc/*.hip into cross_entropy_tv_amd/liblx_ce_tvd.so with hipcc.
Every HIP translation unit is compiled with packed-FP32 instructions disabled
and with IEEE mode off (inputs are finite by contract, and IEEE mode would add
a canonicalising instruction in front of every max).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblx_ce_tvd.so")
SOURCES = ["api.hip", "forward.hip", "forward_cluster.hip", "backward.hip", "reduce.hip", "vocab_parallel.hip",
           "lm_head.hip", "noalloc.hip", "stream.hip"]
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build the library")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object in parallel, then link the shared library."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc(), *HIP_FLAGS, *inc, "-c", os.path.join(HERE, "csrc", src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait() if procs[0][1].poll() is None else None
            import time
            time.sleep(0.05)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(f"--- {src}\n{out}")
        elif out.strip() and verbose:
            print(out)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
