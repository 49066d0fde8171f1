"""Build libusp.so (HIP, gfx950) in-tree.

Usage: ``python -m ulysses_sequence_attention_amd.build [--verbose]``.
Compiles every ``csrc/*.hip`` with hipcc for gfx950 into ``_build/`` at the
repository root and links ``ulysses_sequence_attention_amd/libusp.so``.
Always recompiles, also when a built library is already present. Also
builds the plain C consumers of the ABI under ``tests/c_abi``: one that runs
on the GPU, and a host-only one linked against a copy of the library whose
host code carries the AddressSanitizer (``_build/asan``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libusp.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU ops stay off (the compiler still emits scalar fp32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return r.stdout + r.stderr


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = FLAGS + list(extra_flags or [])
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        for src in sources:
            obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
            objs.append(obj)
            jobs.append(ex.submit(_run, [HIPCC, *flags, "-c", src, "-o", obj], verbose))
        logs = [j.result() for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIB


# Host AddressSanitizer build: the library's host code instrumented (the
# device code is not: every -fsanitize= sits behind -Xarch_host), linked into
# the plain C host check of tests/c_abi, which needs no GPU.
ASAN_BUILD = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_BUILD, "libusp_asan.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "usp_host_check.c")
HOST_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "usp_host_check")


def build_host_check(verbose: bool = False) -> str:
    """Compile libusp with the host AddressSanitizer into _build/asan and the
    host-only C check against it (tests/c_abi/usp_host_check)."""
    os.makedirs(ASAN_BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = FLAGS + ASAN_FLAGS
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        jobs = []
        for src in sources:
            obj = os.path.join(ASAN_BUILD, os.path.basename(src)[:-4] + ".o")
            objs.append(obj)
            jobs.append(ex.submit(_run, [HIPCC, *flags, "-c", src, "-o", obj], verbose))
        for j in jobs:
            j.result()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_FLAGS, "-o", ASAN_LIB, *objs],
         verbose)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    tmp = HOST_CHECK_BIN + ".tmp"
    _run([clang, "-std=c11", "-O1", "-g", "-Wall", *ASAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), HOST_CHECK_SRC, "-o", tmp,
          "-L", ASAN_BUILD, "-lusp_asan", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../../_build/asan", "-Wl,-rpath," + os.path.join(rocm, "lib")], verbose)
    os.replace(tmp, HOST_CHECK_BIN)
    return HOST_CHECK_BIN


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "usp_abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "usp_abi_check")


def build_c_check(verbose: bool = False) -> str:
    """Compile the plain C consumer of the ABI (tests/c_abi) with gcc against
    include/usp.h, libusp.so and the HIP runtime; no PyTorch involved."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    tmp = C_CHECK_BIN + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
          C_CHECK_SRC, "-o", tmp, "-L", PKG, "-lusp", "-L", os.path.join(rocm, "lib"),
          "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../../ulysses_sequence_attention_amd",
          "-Wl,-rpath," + os.path.join(rocm, "lib")], verbose)
    os.replace(tmp, C_CHECK_BIN)
    return C_CHECK_BIN


if __name__ == "__main__":
    extra = [a for a in sys.argv[1:] if a != "--verbose"]
    print(build(verbose="--verbose" in sys.argv, extra_flags=extra))
    print(build_c_check(verbose="--verbose" in sys.argv))
    print(build_host_check(verbose="--verbose" in sys.argv))
