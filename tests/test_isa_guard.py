"""Host-side guard on the generated gfx950 assembly (no GPU needed).

The pipelined kernel programs M0 (the LDS base of a buffer_load ... lds copy)
inside its own inline assembly.  The compiler does not model that write, so
the kernels must not rely on M0 anywhere else: every M0 reference in the
device code has to be the three-instruction copy sequence
``s_mov_b32 m0, sN`` / ``s_nop 0`` / ``buffer_load_dwordx4 ... lds``.
The test compiles the library's device code to assembly with the same flags
as the build and checks exactly that.
"""
import os
import re
import shutil
import subprocess

import pytest

from dense_mixed_precision_amd import build as mpbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "mpgemm.s"
    flags = [f for f in mpbuild.flags() if f not in ("-shared", "-fPIC")]
    cmd = [mpbuild.hipcc(), *flags, "--cuda-device-only", "-S", mpbuild.SRC, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().splitlines()


def _instructions(lines):
    """(index, text) of instruction lines: no labels, directives or comments."""
    out = []
    for i, line in enumerate(lines):
        t = line.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        out.append(t)
    return out


def test_m0_is_only_written_by_the_copy_sequence(device_asm):
    ins = _instructions(device_asm)
    uses = [i for i, t in enumerate(ins) if re.search(r"\bm0\b", t)]
    assert uses, "no LDS copies found in the device code"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i]), f"unexpected M0 use: {ins[i]!r}"
        assert ins[i + 1] == "s_nop 0", f"missing wait state after {ins[i]!r}: {ins[i + 1]!r}"
        assert ins[i + 2].startswith("buffer_load_dwordx4") and ins[i + 2].endswith(" lds"), \
            f"M0 write not followed by an LDS copy: {ins[i + 2]!r}"


def test_no_private_scratch_in_pipelined_kernels(device_asm):
    """The pipelined and narrow kernels (every choice of the factory but the
    fallback) keep all their state in registers and LDS."""
    text = "\n".join(device_asm)
    kernels = [(n, b) for n, b in re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S)
               if "gemm_pipe" in n or "gemm_narrow" in n]
    assert len(kernels) >= 20 and any("gemm_narrow" in n for n, _ in kernels)
    for name, body in kernels:
        size = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
        assert size == 0, f"{name} spills to scratch ({size} bytes)"
