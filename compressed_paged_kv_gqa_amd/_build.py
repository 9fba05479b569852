"""Builds libzp.so in-tree: HIP kernels for gfx950 with hipcc, the host-only
allocator, planner and scheduler with g++, linked into one shared library next to this file.

Usage: ``python -m compressed_paged_kv_gqa_amd._build`` (or ``build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libzp.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the device code (-packed-fp32-ops);
# the host pass of hipcc does not know the feature and says so, harmlessly.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]

HIP_SOURCES = ["zp_decode.hip", "zp_prefill.hip", "zp_score.hip", "zp_select.hip"]
CXX_SOURCES = ["zp_host.cpp", "zp_sched.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # drop the host-pass notice about the device-only target feature
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    """Compiles every source and links libzp.so. Returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    cxx = shutil.which("g++") or "g++"
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([cxx, *CXX_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg:
                print(msg, file=sys.stderr)
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_host_sanitized(out_path):
    """The host-only part of the library (allocator, planner, capacity,
    scheduler) as a separate shared library built with g++ under
    AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests. It
    holds no GPU entry point. Load it with ZP_LIBRARY=<path> and the ASan
    runtime preloaded (``sanitizer_runtime()``)."""
    cxx = shutil.which("g++") or "g++"
    srcs = [os.path.join(CSRC, s) for s in CXX_SOURCES]
    _run([cxx, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", INCLUDE, "-I", CSRC, *srcs, "-o", out_path])
    return out_path


def sanitizer_runtime():
    """Path of g++'s AddressSanitizer runtime (to preload into a Python that
    loads the sanitized host library)."""
    cxx = shutil.which("g++") or "g++"
    return subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
