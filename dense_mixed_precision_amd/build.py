"""Build step for the gfx950 GEMM library (``libmpgemm.so``, in-tree).

``build()`` always recompiles ``csrc/mpgemm.hip`` with hipcc for gfx950.
Packed FP32 VALU instructions are disabled on the device side
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it
does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mpgemm.hip")
DEPS = [SRC, os.path.join(HERE, "csrc", "kernels.hpp"), os.path.join(ROOT, "include", "mpgemm.h")]
LIB = os.path.join(HERE, "libmpgemm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmpgemm.so)")


def flags(extra=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-I", os.path.join(ROOT, "include"),
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *extra]


def build(extra=(), out: str = LIB, verbose: bool = False) -> str:
    """Compile the library to ``out`` (default: in-tree ``libmpgemm.so``)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(extra), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "abi_check")
ROCM = "/opt/rocm"


def build_c_check(verbose: bool = False) -> str:
    """Compile the plain-C caller of the library (a test program: it uses
    only mpgemm.h and the HIP runtime's allocation calls) with gcc, linked
    against the in-tree libmpgemm.so through an $ORIGIN-relative rpath."""
    cc = shutil.which("gcc") or "gcc"
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), C_CHECK_SRC, "-o", C_CHECK_BIN,
           "-L", HERE, "-lmpgemm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../dense_mixed_precision_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    return C_CHECK_BIN


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
