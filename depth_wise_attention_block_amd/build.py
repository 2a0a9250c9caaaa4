"""Compile libattnres.so for gfx950 with hipcc (runs on a host without a GPU).

``python -m depth_wise_attention_block_amd.build`` or ``build()``.  Always
recompiles.  The library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
REPO = os.path.dirname(HERE)
LIB_NAME = "libattnres.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PATTERN_BENCH = os.path.join(HERE, "pattern_bench")
# host-only C ABI (argument checks, range arithmetic, store bookkeeping) under
# AddressSanitizer + UndefinedBehaviorSanitizer, with launchers that launch
# nothing: the CPU tests run the binding's host checks against it
HOSTSAN_LIB = os.path.join(HERE, "libattnres_hostsan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
CAPI_CLIENT = os.path.join(HERE, "capi_client")
SOURCES = ("aggregate.hip", "accumulate.hip", "twophase.hip", "backward.hip", "capi.cpp")
ARCH = "gfx950"

# -packed-fp32-ops: never emit packed fp32 arithmetic; the host pass warns that
# it does not know the feature, which is harmless.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP/C++ source into ``libattnres.so``; returns its path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-shared", "-I", os.path.join(REPO, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    log = "\n".join(l for l in proc.stdout.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{log}")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, LIB_PATH)
    _compile([hipcc(), *HIP_FLAGS, *extra_flags, os.path.join(CSRC, "pattern_bench.hip")], PATTERN_BENCH, verbose)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    build_host_sanitized(rocm, verbose)
    # a plain C program that calls the library through the header alone
    _compile([shutil.which("gcc") or "gcc", "-std=c11", "-O2", "-Wall", "-I", os.path.join(REPO, "include"),
              "-I", os.path.join(rocm, "include"), os.path.join(CSRC, "capi_client.c"), "-L", HERE, "-lattnres",
              "-Wl,-rpath,$ORIGIN", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
              "-Wl,-rpath," + os.path.join(rocm, "lib")], CAPI_CLIENT, verbose)
    return LIB_PATH


def build_host_sanitized(rocm: str, verbose: bool = False) -> str:
    """capi.cpp + host_stubs.cpp with g++ (host code only, no .hip file) under
    ASan/UBSan -> libattnres_hostsan.so.  Load it with the ASan runtime
    preloaded (``sanitizer_env()``)."""
    _compile([shutil.which("g++") or "g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SAN_FLAGS,
              "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(REPO, "include"), "-I", CSRC,
              "-I", os.path.join(rocm, "include"), os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "host_stubs.cpp"),
              "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")],
             HOSTSAN_LIB, verbose)
    return HOSTSAN_LIB


def sanitizer_env(base=None) -> dict:
    """Environment for a child process that loads libattnres_hostsan.so: the
    binding pointed at it, the gcc ASan runtime loaded first (ahead of whatever
    the environment already preloads), leak checking off (the Python process
    itself is not instrumented), any report fatal."""
    env = dict(os.environ if base is None else base)
    gcc = shutil.which("gcc") or "gcc"
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    env["LD_PRELOAD"] = (asan + " " + env["LD_PRELOAD"]).strip() if env.get("LD_PRELOAD") else asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["ATTNRES_LIBRARY"] = HOSTSAN_LIB
    return env


def _compile(cmd, target: str, verbose: bool) -> None:
    tmp = target + f".tmp{os.getpid()}"
    cmd = [*cmd, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    log = "\n".join(l for l in proc.stdout.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed ({proc.returncode}):\n{log}")
    os.replace(tmp, target)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
