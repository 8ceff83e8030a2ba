"""Build libcsa2.so (the CSA2 HIP library) in-tree for gfx950 with hipcc.

Usage:  python -m hierarchical_kv_indexer_amd.build              the library
        python -m hierarchical_kv_indexer_amd.build --hostcheck  the host-code sanitizer check:
            every source with AddressSanitizer and UndefinedBehaviorSanitizer on its host code
            only (device code is built as usual), linked with tests/hostcheck/abi_check.cpp into
            _build/hostcheck/abi_check, a program that exercises the C ABI's host code on a
            machine without a GPU (tests/test_hostcheck.py runs it)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa2.so")
SOURCES = ("scan.hip", "select.hip", "attn.hip", "kvquant.hip", "encoder.hip", "api.cpp", "noalloc.hip")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # no packed fp32 instructions (v_pk_*_f32) in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa2.so)")


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libcsa2.so next to this file; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


HOSTCHECK_DIR = os.path.join(BUILD_DIR, "hostcheck")
HOSTCHECK_BIN = os.path.join(HOSTCHECK_DIR, "abi_check")
# sanitizers on the host code only: each flag goes to the host compilation through -Xarch_host
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_hostcheck(verbose: bool = False) -> str:
    """The sanitized host-code check program (see the module docstring); returns its path."""
    os.makedirs(HOSTCHECK_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, HOSTCHECK_DIR, HOST_SANITIZE), SOURCES))
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    san = "-fsanitize=" + ",".join(("address", "undefined"))
    drv = os.path.join(ROOT, "tests", "hostcheck", "abi_check.cpp")
    cmd = [clang, "-O1", "-g", "-std=c++17", san, "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", "/opt/rocm/include", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", HOSTCHECK_BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hostcheck link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {HOSTCHECK_BIN}")
    return HOSTCHECK_BIN


if __name__ == "__main__":
    if "--hostcheck" in sys.argv[1:]:
        build_hostcheck(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
