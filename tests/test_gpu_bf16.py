"""GPU parity for BF16 inputs (the other 16-bit tensor-core input type of
"Tensor cores with WMMA", section "A warp owns a tile, and no thread owns an
element"): the BF16 entry points through the C ABI against the CPU oracle's
BF16 product on the same bit patterns, in every storage order.

Acceptance: |C_gpu - C_ref| <= 1e-3 * sum_k |a_ik b_kj| + 1e-5 elementwise;
small integers (exact in BF16) must match bit for bit.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, freivalds_ok, run_layout, stored

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]


def oracle_bf16(A, B, C0, alpha, beta, la, lb):
    return oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)), None if C0 is None else C0.numpy(),
                       alpha, beta, layout_a=la, layout_b=lb, in_type="bf16")


def full_check(label, A, B, C0, alpha, beta, la, lb, **kw):
    got, gC = run_layout(A, B, C0, alpha, beta, la, lb, **kw)
    ref, absdot = oracle_bf16(A, B, C0, alpha, beta, la, lb)
    assert_close(label, got, ref, absdot, K=A.shape[1], alpha=alpha, beta=beta, C0=C0)
    assert gC.untouched_outside_window(), f"{label}: wrote outside the M x N window"


def _bf16_ids():
    # the narrow entries (N <= 16 only) have their own tests
    return [i for i in range(mp.mpgemm_num_configs())
            if mp.mpgemm_config_info(i)["in_type"] == mp.MPGEMM_IN_BF16
            and mp.mpgemm_config_info(i)["kind_name"] != "narrow"]


SHAPES = [(1, 1, 1), (17, 15, 33), (65, 63, 129), (611, 613, 617), (300, 17, 40), (4096, 16, 256)]


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_factory_edge_shapes(la, lb, M, N, K):
    A, B, C = make_inputs(M, N, K, "uniform", seed=M + 5 * N + 3 * K + la + 2 * lb, c_init="uniform",
                          dtype=BF16)
    print(f"[bf16 {la}{lb}] {M}x{N}x{K}", flush=True)
    full_check(f"bf16 {la}{lb} {M}x{N}x{K} beta=0", A, B, None, 1.0, 0.0, la, lb)
    full_check(f"bf16 {la}{lb} {M}x{N}x{K} beta=.5", A, B, C, 1.5, 0.5, la, lb)


@pytest.mark.parametrize("cfg", _bf16_ids())
def test_every_bf16_config_ragged_strided(cfg):
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    M, N, K = 261, 147, 101
    lda = 272 if la else 112
    ldb = 112 if lb else 160
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg + 500, c_init="uniform", dtype=BF16)
    print(f"[config {cfg}] bf16 layout {la}{lb} {c['kind_name']}", flush=True)
    full_check(f"config {cfg}", A, B, C, 1.25, -0.75, la, lb, config=cfg, lda=lda, ldb=ldb, ldc=151)


@pytest.mark.parametrize("cfg", [i for i in _bf16_ids() if mp.mpgemm_config_info(i)["kind_name"] == "pipe"])
def test_every_bf16_config_multi_tile_bitwise(cfg):
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    M, N, K = 520, 600, 392
    A, B, _ = make_inputs(M, N, K, "smallint", seed=cfg + 600, dtype=BF16)
    got, _ = run_layout(A, B, None, 1.0, 0.0, la, lb, config=cfg)
    ints = A.to(torch.int64) @ B.to(torch.int64)
    assert np.array_equal(got, ints.numpy().astype(np.float32)), f"config {cfg}: not bitwise"


def test_wide_exponent_range():
    """BF16 keeps FP32's exponent range: operands near 2^+-60 must come
    through the matrix cores and the epilogue unscaled."""
    M, N, K = 96, 80, 200
    A, B, _ = make_inputs(M, N, K, "uniform", seed=71, dtype=torch.float32)
    A = (A.float() * 2.0 ** 60).to(BF16)
    B = (B.float() * 2.0 ** -61).to(BF16)
    full_check("bf16 scaled", A, B, None, 1.0, 0.0, 0, 0)


def test_2048_every_element_and_freivalds():
    M = N = K = 2048
    A, B, _ = make_inputs(M, N, K, "uniform", seed=1101, dtype=BF16)
    got, _ = run_layout(A, B, None, 1.0, 0.0, 0, 0)
    assert np.all(np.isfinite(got))
    ref, absdot = oracle.gemm(bits(A), bits(B), None, 1.0, 0.0, in_type="bf16")
    assert_close("2048 bf16", got, ref, absdot, K=K, alpha=1.0)
    ok, ratio = freivalds_ok(got, A.float(), B.float(), None, 1.0, 0.0, seed=9)
    assert ok, f"Freivalds failed (worst {ratio:.3g})"
