"""Build the gfx950 libraries in-tree with hipcc:

    libssmscan.so  -- the scan kernels and their C ABI (include/ssm_scan.h)
    libssmbench.so -- the benchmark's measurement helpers (include/ssm_bench.h)

    python -m selective_scan_ssm_amd.build

Every call recompiles all sources (objects go to selective_scan_ssm_amd/_build/).
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssmscan.so")
BENCH_LIB = os.path.join(PKG, "libssmbench.so")
ARCH = "gfx950"

SOURCES = ["scan_fwd.hip", "scan_rows_bf16.hip", "scan_rows_f32.hip", "scan_rows_2d_bf16.hip",
           "scan_rows_2d_f32.hip", "scan_general_bf16.hip", "scan_general_bf16_xf32.hip", "scan_general_f32.hip",
           "sm1_scan.hip", "state_update.hip", "scan_bwd.hip", "conv1d.hip", "scan_2d.hip",
           "ssd_scan.hip", "dt_proj.hip", "scan_noalloc.hip", "ssm_abi.cpp"]
BENCH_SOURCES = ["microbench.hip"]

# Packed fp32 VALU forms are switched off (plain fp32 VALU only); code object
# v5 is what the HIP runtime shipped with torch loads.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], BENCH_LIB, verbose)
    return LIB


def build_host_sanitized(out: str) -> str:
    """libssmscan.so with its host-side C ABI (argument validation, aliasing
    and size arithmetic, ssm_abi.cpp) compiled under AddressSanitizer and
    UndefinedBehaviorSanitizer; the kernels' objects are the regular ones
    (GPU code is not sanitized: -fsanitize goes to the host pass only)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.basename(src) + ".o") for src in SOURCES if src != "ssm_abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    abi_obj = os.path.join(BUILD, "ssm_abi.cpp.asan.o")
    cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, *san, "-c", os.path.join(CSRC, "ssm_abi.cpp"), "-o", abi_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized ssm_abi.cpp:\n{r.stdout}\n{r.stderr}")
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, abi_obj,
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the sanitized library failed:\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
