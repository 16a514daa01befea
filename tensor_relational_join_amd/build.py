"""Build libja.so (host core + HIP kernels for gfx950) in-tree with hipcc.

    python -m tensor_relational_join_amd.build [--debug]

Objects go to _build/ at the repository root; the library lands next to this
file as libja.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libja.so")
BUILD = os.path.join(ROOT, "_build")

HOST_SOURCES = ["host/core.cpp", "host/plan.cpp", "host/plan_contract.cpp", "host/repart.cpp", "host/djoin.cpp", "host/planner.cpp", "host/dattn.cpp", "host/calib.cpp"]
HIP_SOURCES = ["hip/gemm.hip", "hip/attention.hip", "hip/stream_ops.hip", "hip/join.hip", "hip/dattn.hip", "hip/calib.hip", "hip/noalloc.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]
# gfx950 only; packed-fp32 instructions are disabled in all device code.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, extra) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    is_hip = src.endswith(".hip")
    cmd = [_hipcc()] + COMMON + list(extra) + (DEVICE + ["-x", "hip"] if is_hip else ["-D__HIP_PLATFORM_AMD__"])
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-g"] if debug else []
    srcs = HOST_SOURCES + HIP_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(debug="--debug" in sys.argv, verbose=True)
