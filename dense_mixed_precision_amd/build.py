"""Build step for the gfx950 GEMM libraries (in-tree).

``build()`` always recompiles, with hipcc for gfx950:

* ``libmpgemm.so`` -- the product library (``csrc/mpgemm.hip``, C ABI in
  ``include/mpgemm.h``): the config entries the factory chooses from and the
  fallbacks;
* ``libmpgemm_probes.so`` -- the diagnostics (``csrc/probes.hip``, C ABI in
  ``include/mpgemm_probes.h``);
* ``libmpgemm_timeline.so`` -- the product library built with
  ``-DMPGEMM_TIMELINE``: the same entry points and results, plus the
  per-workgroup timeline of ``include/mpgemm_timeline.h`` (diagnostics);
* with ``candidates=True`` also ``libmpgemm_candidates.so``: the product
  library plus the alternative tile shapes of tile sweeps
  (``-DMPGEMM_CANDIDATES``), which the factory never picks.

Packed FP32 VALU instructions are disabled on the device side
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know the feature, which is harmless.

    python -m dense_mixed_precision_amd.build [--candidates]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SRC = os.path.join(CSRC, "mpgemm.hip")
PROBES_SRC = os.path.join(CSRC, "probes.hip")
DEPS = [SRC, os.path.join(CSRC, "kernels.hpp"), os.path.join(ROOT, "include", "mpgemm.h")]
LIB = os.path.join(HERE, "libmpgemm.so")
PROBES_LIB = os.path.join(HERE, "libmpgemm_probes.so")
CANDIDATES_LIB = os.path.join(HERE, "libmpgemm_candidates.so")
TIMELINE_LIB = os.path.join(HERE, "libmpgemm_timeline.so")
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


def _start(src, out, extra, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(extra), src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), tmp, out


def _finish(job):
    proc, tmp, out = job
    stdout, stderr = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}) for {out}:\n{stdout}\n{stderr}")
    os.replace(tmp, out)
    return out


def build(extra=(), out: str = LIB, verbose: bool = False, probes: bool = True,
          candidates: bool = False) -> str:
    """Compile the product library to ``out`` (default: in-tree
    ``libmpgemm.so``), the diagnostics libraries (probes, timeline), and
    optionally the candidates library, in parallel.  Returns ``out``."""
    jobs = [_start(SRC, out, extra, verbose)]
    if probes:
        jobs.append(_start(PROBES_SRC, PROBES_LIB, extra, verbose))
        jobs.append(_start(SRC, TIMELINE_LIB, (*extra, "-DMPGEMM_TIMELINE"), verbose))
    if candidates:
        jobs.append(_start(SRC, CANDIDATES_LIB, (*extra, "-DMPGEMM_CANDIDATES"), verbose))
    errors = []
    for job in jobs:
        try:
            _finish(job)
        except RuntimeError as e:
            errors.append(str(e))
    if errors:
        raise RuntimeError("\n".join(errors))
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
    print(build(verbose=True, candidates="--candidates" in sys.argv[1:]))
