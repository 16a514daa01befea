"""Build libja.so (host core + HIP kernels for gfx950) in-tree with hipcc.

    python -m tensor_relational_join_amd.build [--debug]
    python -m tensor_relational_join_amd.build --sanitize [--check]

Objects go to _build/ at the repository root; the library lands next to this
file as libja.so.  --sanitize builds libja_asan.so instead: the host core
(planner, join, repartition atoms, ABI validation) with AddressSanitizer and
UndefinedBehaviorSanitizer, the HIP sources as usual (the sanitizers apply to
host code only).  --check then runs the CPU test suite's host, ABI, planner
and buffer-check tests against it (JA_LIBJA names the library, the ASan
runtime is preloaded into the interpreter, leak checking is off because the
interpreter itself is not instrumented); any sanitizer report fails the run.
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


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, src.replace("/", "_") + ".o")
    is_hip = src.endswith(".hip")
    cmd = [_hipcc()] + COMMON + list(extra) + (DEVICE + ["-x", "hip"] if is_hip else ["-D__HIP_PLATFORM_AMD__"])
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


# host-only sanitizer flags: each -fsanitize= behind -Xarch_host, so no device code is built with them
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-fno-omit-frame-pointer",
            "-g", "-O1"]
ASAN_OUT = os.path.join(PKG, "libja_asan.so")


def _generate(build_dir: str) -> str:
    """Write the generated sources (the contraction's assembly K loop) into build_dir/gen."""
    gen = os.path.join(build_dir, "gen")
    os.makedirs(gen, exist_ok=True)
    cmd = [sys.executable, os.path.join(CSRC, "hip", "gen_gemm_asm.py"), os.path.join(gen, "gemm_asm.inc")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("generation failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return gen


def build(debug: bool = False, verbose: bool = False, sanitize: bool = False) -> str:
    build_dir = os.path.join(BUILD, "asan") if sanitize else BUILD
    os.makedirs(build_dir, exist_ok=True)
    extra = (["-g"] if debug else []) + ["-I" + _generate(build_dir)]
    srcs = HOST_SOURCES + HIP_SOURCES

    def one(src):
        return _compile(src, extra + (SANITIZE if sanitize and src in HOST_SOURCES else []), build_dir)

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    out = ASAN_OUT if sanitize else OUT
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def check_sanitized() -> int:
    """The CPU host, ABI, planner and buffer-check tests against
    libja_asan.so; returns the test run's exit status (nonzero on any
    sanitizer report)."""
    rt = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    env = dict(os.environ, JA_LIBJA=ASAN_OUT, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_host.py", "test_abi.py", "test_planner.py",
                                                      "test_device_checks.py")]
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + tests,
                          env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    san = "--sanitize" in sys.argv
    build(debug="--debug" in sys.argv, verbose=True, sanitize=san)
    if san and "--check" in sys.argv:
        sys.exit(check_sanitized())
