"""Build libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_mixture_experts_22_amd.build        # or __graft_entry__.build()

Every source is compiled with hipcc for gfx950 only; objects go to _build/ at
the repository root, the shared library next to this file.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["route.hip", "gemm_prefill.hip", "gemm_packed.hip", "gemm_skinny.hip", "quant4.hip", "misc.hip",
           "validate.hip", "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from forming packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (the C-ABI
# layer and every launcher; device code is compiled as usual).  Each sanitizer
# flag applies to the host compilation only.
SANITIZE_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_BUILD = os.path.join(BUILD, "sanitized")
SAN_LIB = os.path.join(SAN_BUILD, "libmoe_sanitized.so")


# Tile-trace build: the same library with per-tile timestamps in the packed
# grouped GEMMs (include/moe_tile_trace.h), read by tile_trace.py.
TRACE_BUILD = os.path.join(BUILD, "tiletrace")
TRACE_LIB = os.path.join(PKG, "libmoe_tiletrace.so")


def _compile(src: str, sanitize: bool = False, trace: bool = False) -> str:
    out_dir = SAN_BUILD if sanitize else (TRACE_BUILD if trace else BUILD)
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = compile_flags() + (SANITIZE_FLAGS if sanitize else []) + (["-DMOE_TILE_TRACE"] if trace else [])
    cmd = [hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_tile_trace(verbose: bool = True) -> str:
    """libmoe_tiletrace.so next to libmoe.so: every source compiled with
    MOE_TILE_TRACE (only the packed grouped GEMMs and the C ABI change)."""
    os.makedirs(TRACE_BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, trace=True), SOURCES))
    tmp = TRACE_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, TRACE_LIB)
    if verbose:
        print(f"built {TRACE_LIB}")
    return TRACE_LIB


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized build links (a process
    that did not start with it must preload it)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cands = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not cands:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return cands[-1]


def build_sanitized(verbose: bool = True) -> str:
    """libmoe_sanitized.so: the same sources with host-side ASan + UBSan.  The
    objects are linked by the host compiler driver (they carry their device
    code already)."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize=True), SOURCES))
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    clangxx = os.path.join(rocm, "llvm", "bin", "clang++")
    host_link = [clangxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", "-o", SAN_LIB,
                 *objs, "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    res = subprocess.run(host_link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
