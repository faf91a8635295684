"""Build libqkv.so in-tree with hipcc for gfx950.

Usage: python -m video_model_kv_amd.build   (or call build()).  Every call
recompiles.  The HIP flags keep IEEE semantics: no fast-math, no contraction of
separate multiplies and adds, correctly rounded fp32 division, and no packed
fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqkv.so")
HIP_SOURCES = ["kmeans.hip", "quant.hip", "attend.hip", "gram.hip", "eigh.hip", "scratch.hip", "temporal.hip"]
CPP_SOURCES = ["qkv_host.cpp", "timing.cpp"]
ARCH = os.environ.get("QKV_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["hipcc", *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["hipcc", "-O2", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}", *inc,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + CPP_SOURCES]
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, "-lpthread"])
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
