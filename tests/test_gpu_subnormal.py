"""Subnormal inputs through the matrix instructions, exactly.

The gate of "Capstone 4: a tensor-core GEMM" (section "Independent gate")
has an adversarial case with edge values, subnormals among them.  Within the
acceptance rule a kernel that flushed subnormal inputs to zero could still
pass when large values sit in the same rows, so here the data make every
product and every partial sum exact in FP32 and the result must equal the
oracle's bit for bit:

* FP16: one operand holds subnormals n * 2^-24 (n in 1..1023, mixed signs),
  the other small integers in [-2, 2].  Every product is an integer multiple
  of 2^-24 below 2^-12 and every partial sum a multiple of 2^-24 below
  K * 2046 * 2^-24 < 1, which FP32 holds exactly.
* BF16: one operand holds subnormals n * 2^-133 (n in 1..127), the other
  +-2^110 or +-2^111, so every product is a normal FP32 number n * 2^-23 or
  n * 2^-22 and every partial sum a multiple of 2^-23 well inside FP32's
  24-bit significand.

A flushed input changes the sum by at least 2^-24 (FP16) or 2^-23 (BF16),
which a bitwise comparison sees.  Every entry of the table runs it in its
input format and storage orders (a K tail included), through the C ABI.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits
from tests.gpu_util import run_layout, stored

pytestmark = pytest.mark.gpu


def subnormal_f16(shape, rng):
    n = rng.integers(1, 1024, shape) * rng.choice([-1, 1], shape)
    x = torch.from_numpy((n * 2.0 ** -24).astype(np.float32)).to(torch.float16)
    assert np.all(np.abs(bits(x).astype(np.int64) & 0x7C00) == 0)        # exponent field 0: subnormal
    return x


def small_int(shape, rng, dtype):
    return torch.from_numpy(rng.integers(-2, 3, shape).astype(np.float32)).to(dtype)


def subnormal_bf16(shape, rng):
    n = rng.integers(1, 128, shape) * rng.choice([-1, 1], shape)
    x = torch.from_numpy((n * 2.0 ** -133).astype(np.float32)).to(torch.bfloat16)
    assert np.all((bits(x).astype(np.int64) & 0x7F80) == 0)              # exponent field 0: subnormal
    return x


def big_pow2_bf16(shape, rng):
    e = rng.integers(110, 112, shape)
    return torch.from_numpy((rng.choice([-1.0, 1.0], shape) * np.exp2(e.astype(np.float64))).astype(np.float32)).to(
        torch.bfloat16)


def _entries():
    out = []
    for i in range(mp.mpgemm_num_configs()):
        c = mp.mpgemm_config_info(i)
        if c["kind_name"] in ("pipe", "narrow", "direct"):
            out.append(i)
    return out


@pytest.mark.parametrize("sub_side", ["A", "B"])
@pytest.mark.parametrize("cfg", _entries())
def test_subnormal_inputs_bitwise(cfg, sub_side):
    c = mp.mpgemm_config_info(cfg)
    bf16 = c["in_type"] == mp.MPGEMM_IN_BF16
    la, lb = c["layout_a"], c["layout_b"]
    M, N, K = (520, 13, 397) if c["kind_name"] == "narrow" else (520, 600, 397)
    rng = np.random.default_rng(cfg * 2 + (sub_side == "B"))
    if bf16:
        sub, other = subnormal_bf16, big_pow2_bf16
    else:
        sub = subnormal_f16
        other = lambda shape, r: small_int(shape, r, torch.float16)  # noqa: E731
    A = sub((M, K), rng) if sub_side == "A" else other((M, K), rng)
    B = sub((K, N), rng) if sub_side == "B" else other((K, N), rng)
    print(f"[config {cfg} {c['kind_name']} {'bf16' if bf16 else 'f16'} {la}{lb}] subnormal {sub_side}", flush=True)
    got, gC = run_layout(A, B, None, 1.0, 0.0, la, lb, config=cfg)
    ref, _ = oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)), layout_a=la, layout_b=lb,
                         in_type="bf16" if bf16 else "f16")
    assert np.all(ref != 0) or np.count_nonzero(ref) > 0.9 * ref.size
    assert np.array_equal(got, ref.astype(np.float32)), \
        f"config {cfg}: not bitwise ({np.count_nonzero(got != ref.astype(np.float32))} entries differ)"
    assert gC.untouched_outside_window()
