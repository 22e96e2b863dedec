"""Build liborca.so in-tree: hipcc for the gfx950 kernels and the engine,
g++ for the host-only allocator and scheduler.

    python -m orca_selective_iteration_amd.build

Every call recompiles every source.  No GPU is needed (hipcc cross-compiles
for gfx950).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liborca.so")

HIP_SOURCES = ["ln.hip", "gemm.hip", "attn.hip", "engine.hip"]
CPP_SOURCES = ["status.cpp", "kv.cpp", "sched.cpp"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-munsafe-fp-atomics",
    # packed fp32 instructions are kept out of all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link liborca.so; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    steps = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src),
                      "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, steps))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [s[-1] for s in steps]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    # a kernel whose host-side launch stub failed to instantiate leaves an
    # undefined symbol that only shows when the library is loaded
    import ctypes
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load: {e}")
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "liborca_host_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build_host_sanitized() -> str:
    """The host-only part of the library (status, K/V allocator, scheduler)
    built with AddressSanitizer and UndefinedBehaviorSanitizer, for running
    the host tests against it (ORCA_LIB / ORCA_HOST_ONLY, see lib.py).  CPU
    code only: g++, no HIP source.  Returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    gxx = shutil.which("g++") or "g++"
    objs = []
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".san.o")
        _run([gxx, *SAN_FLAGS, "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    _run([gxx, *SAN_FLAGS, "-shared", "-o", SAN_LIB, *objs])
    return SAN_LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
