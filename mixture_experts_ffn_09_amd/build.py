"""Build ``libmoe_ffn.so`` (HIP, gfx950) in place.

    python -m mixture_experts_ffn_09_amd.build [--jobs N] [--sanitized]

Every source in ``csrc/`` is compiled with hipcc for gfx950 and linked into
one shared library next to this file.  Always rebuilds.  --sanitized also
builds a copy whose host code is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer (``_build/sanitized/``, for CPU tests).
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_ffn.so")
SOURCES = ["abi.cpp", "router.hip", "permute.hip", "ffn_stream.hip", "ffn_gemm.hip",
           "ffn_f32.hip", "combine.hip", "pack.hip", "stats.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # no packed float32 arithmetic in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_DIR = os.path.join(BUILD, "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libmoe_ffn.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """The library with its host code (the C ABI's argument checks, workspace
    carving and launch set-up in abi.cpp) built with AddressSanitizer and
    UndefinedBehaviorSanitizer, for CPU tests of the validation layer.  The
    sanitizers apply to host code only (-Xarch_host); the device objects are
    the regular ones.  Load it with the clang ASan runtime preloaded."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    abi = os.path.join(SAN_DIR, "abi.cpp.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-g"]
    cmd = [HIPCC, *FLAGS, *san, "-x", "hip", "-c", os.path.join(CSRC, "abi.cpp"), "-o", abi]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on abi.cpp (sanitized):\n{r.stderr}")
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", SAN_LIB, abi, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime to preload."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--sanitized", action="store_true")
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    if a.sanitized:
        build_host_sanitized(verbose=True)
    sys.exit(0)
