"""GPU parity for the per-column bias epilogue (the position-dependent
epilogue of "Tensor cores with WMMA", section "The habit this API takes
away"), through mpgemm_gemm_ex against the oracle's biased product:

    C[i][j] <- alpha * sum_k A[i][k] B[k][j] + beta * C[i][j] + bias[j]

Every kernel kind adds the bias: the pipelined kernels, the narrow kernel,
the direct fallback and the scale-only path (alpha == 0 or
K == 0).  Acceptance: |C_gpu - C_ref| <= 1e-3 * sum_k |a_ik b_kj| + 1e-5;
the bias (|bias| <= 2 here) is added once in FP32, a rounding of at most
2^-24 of the result, far inside the absolute term.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, run_layout, stored

pytestmark = pytest.mark.gpu


def _bias(N, seed):
    return np.random.default_rng(seed).uniform(-2, 2, N).astype(np.float32)


def check(label, A, B, C0, alpha, beta, la, lb, bias, **kw):
    in_type = "bf16" if A.dtype == torch.bfloat16 else "f16"
    got, gC = run_layout(A, B, C0, alpha, beta, la, lb, bias=bias, **kw)
    ref, absdot = oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)),
                              None if C0 is None else C0.numpy(), alpha, beta,
                              layout_a=la, layout_b=lb, in_type=in_type, bias=bias)
    assert_close(label, got, ref, absdot, K=A.shape[1], alpha=alpha, beta=beta, C0=C0, bias=bias)
    assert gC.untouched_outside_window(), f"{label}: wrote outside the M x N window"


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("la,lb", [(0, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (17, 15, 33), (611, 613, 617), (300, 17, 40),
                                   (1024, 1024, 256)])
def test_factory_with_bias(dtype, la, lb, M, N, K):
    A, B, C = make_inputs(M, N, K, "uniform", seed=M + N + K + la + 2 * lb, c_init="uniform", dtype=dtype)
    bias = _bias(N, M + K)
    print(f"[bias {dtype} {la}{lb}] {M}x{N}x{K}", flush=True)
    check(f"{M}x{N}x{K} beta=0", A, B, None, 1.0, 0.0, la, lb, bias)
    check(f"{M}x{N}x{K} beta=.5", A, B, C, 1.5, 0.5, la, lb, bias)


def _configs_for(in_type, la, lb):
    out = []
    for i in range(mp.mpgemm_num_configs()):
        c = mp.mpgemm_config_info(i)
        if c["kind_name"] in ("scale", "narrow"):    # narrow: N <= 16, its own bias test
            continue
        if c["in_type"] == in_type and (c["layout_a"], c["layout_b"]) == (la, lb):
            out.append(i)
    return out


@pytest.mark.parametrize("cfg", _configs_for(mp.MPGEMM_IN_F16, 0, 0) + _configs_for(mp.MPGEMM_IN_BF16, 1, 0))
def test_every_kernel_adds_the_bias(cfg):
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    dtype = torch.bfloat16 if c["in_type"] == mp.MPGEMM_IN_BF16 else torch.float16
    M, N, K = 261, 147, 101
    lda = 272 if la else 112
    ldb = 112 if lb else 160
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg + 700, c_init="uniform", dtype=dtype)
    check(f"config {cfg}", A, B, C, 1.25, -0.75, la, lb, _bias(N, cfg), config=cfg, lda=lda, ldb=ldb,
          ldc=151)


def test_scale_path_adds_the_bias_and_does_not_read_C_when_beta_is_zero():
    M, N = 130, 70
    bias = _bias(N, 3)
    A, B, C = make_inputs(M, N, 33, "uniform", seed=3, c_init="uniform")
    got, _ = run_layout(A, B, C, 0.0, 0.5, 0, 0, bias=bias)         # alpha == 0
    assert np.array_equal(got, np.float32(0.5) * C.numpy() + bias[None, :])
    A0, B0, _ = make_inputs(M, N, 0, "uniform", seed=3)
    got, _ = run_layout(A0, B0, None, 1.0, 0.0, 0, 0, bias=bias)    # K == 0, NaN-poisoned C
    assert np.array_equal(got, np.broadcast_to(bias, (M, N)))


def test_bias_validation():
    dev = torch.device("cuda:0")
    A = torch.zeros(8, 8, dtype=torch.float16, device=dev)
    C = torch.zeros(8, 8, device=dev)
    with pytest.raises(ValueError):
        mp.gemm(A, A, C, bias=torch.zeros(7, device=dev))
    b = torch.zeros(9, device=dev)
    rc = mp.mpgemm_gemm_ex(0, 0, 0, 8, 8, 8, A.data_ptr(), 8, A.data_ptr(), 8, C.data_ptr(), 8,
                           1.0, 0.0, b.data_ptr() + 2, 0)
    assert rc == mp.MPGEMM_EALIGN
    rc = mp.mpgemm_gemm_ex(2, 0, 0, 8, 8, 8, A.data_ptr(), 8, A.data_ptr(), 8, C.data_ptr(), 8,
                           1.0, 0.0, 0, 0)
    assert rc == mp.MPGEMM_ETYPE
