"""GPU parity of the narrow kernel (N <= 16, A row-major; the "skinny" shape of
"Capstone 4: a tensor-core GEMM", section "Independent gate"), through the C
ABI's forced-config entry points, against the oracle.

Every narrow table entry (FP16/BF16, B row- or column-major, each load
depth) on ragged M, N from 1 to 16, K below 8 (the tail alone), K with and
without a tail, K spanning many k-steps per wave and fewer k-steps than
waves; operands padded past their rows with a NaN pattern; exact small
integers bit for bit, uniform inputs with beta != 0 within tolerance; a
bias; and the entry refusing N > 16 or a column-major A.  A one-column B
stored column-major (which the tensor binding sees as row-major) goes
through the C ABI directly.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import Guarded, assert_close, device, run_layout, stored

pytestmark = pytest.mark.gpu


def _narrow_ids():
    return [i for i in range(mp.mpgemm_num_configs()) if mp.mpgemm_config_info(i)["kind_name"] == "narrow"]


SHAPES = [(16, 16, 32), (17, 1, 5), (33, 7, 1), (255, 16, 64), (513, 9, 1031), (1000, 13, 617),
          (1000, 16, 616), (4096, 16, 4096), (40, 16, 8200)]


def run_abi(A, B, C0, alpha, beta, la, lb, config, lda, ldb, ldc=None):
    """Like run_layout, through mpgemm_gemm_ex_with_config with raw device
    pointers: A row-major, B stored in order `lb`, guarded buffers."""
    assert la == 0
    M, K = A.shape
    N = B.shape[1]
    gA = Guarded(A, ld=lda)
    gB = Guarded(stored(B, lb), ld=ldb)
    if C0 is None:
        gC = Guarded(torch.zeros((M, N), dtype=torch.float32), ld=ldc, fill=float("nan"))
    else:
        gC = Guarded(C0, ld=ldc)
    in_type = mp.MPGEMM_IN_BF16 if A.dtype == torch.bfloat16 else mp.MPGEMM_IN_F16

    def ptr(g):
        return g.flat.data_ptr() + g.start * g.flat.element_size()

    rc = mp.mpgemm_gemm_ex_with_config(config, in_type, 0, lb, M, N, K, ptr(gA), gA.ld, ptr(gB), gB.ld, ptr(gC),
                                       gC.ld, alpha, beta, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == mp.MPGEMM_OK, mp.mpgemm_strerror(rc)
    torch.cuda.synchronize()
    return gC.result(), gC


def _ref(A, B, C0, alpha, beta, lb, fmt, bias=None):
    return oracle.gemm(bits(A), bits(stored(B, lb)), None if C0 is None else C0.numpy(), alpha, beta,
                       layout_b=lb, in_type=fmt, bias=bias)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("cfg", _narrow_ids())
def test_narrow_config(cfg, M, N, K):
    c = mp.mpgemm_config_info(cfg)
    lb = c["layout_b"]
    # A one-column B describes the same bytes in either storage order, and
    # the tensor binding passes it as row-major; the column-major entries
    # are called through the C ABI directly for it.
    runner = run_abi if (lb and N == 1) else run_layout
    fmt = "bf16" if c["in_type"] == mp.MPGEMM_IN_BF16 else "f16"
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    lda, ldb = K + 3, (K if lb else N) + 5
    A, B, _ = make_inputs(M, N, K, "smallint", seed=cfg * 13 + M + N + K, dtype=dtype)
    got, gC = runner(A, B, None, 1.0, 0.0, 0, lb, config=cfg, lda=lda, ldb=ldb)
    ref, _ = _ref(A, B, None, 1.0, 0.0, lb, fmt)
    assert np.array_equal(got, ref.astype(np.float32)), f"config {cfg} {M}x{N}x{K}: not bitwise"
    assert gC.untouched_outside_window()
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg * 17 + M + N + K, c_init="uniform", dtype=dtype)
    got, gC = runner(A, B, C, 1.5, 0.5, 0, lb, config=cfg, lda=lda, ldb=ldb, ldc=N + 2)
    ref, absdot = _ref(A, B, C, 1.5, 0.5, lb, fmt)
    assert_close(f"config {cfg} {M}x{N}x{K} beta=.5", got, ref, absdot, K=K, alpha=1.5, beta=0.5, C0=C)
    assert gC.untouched_outside_window()


@pytest.mark.parametrize("M,N,K", [(40, 1, 5), (40, 3, 12), (70, 7, 40), (70, 9, 33), (100, 13, 617),
                                   (33, 16, 9)])
@pytest.mark.parametrize("cfg", [i for i in _narrow_ids() if mp.mpgemm_config_info(i)["layout_b"] == 0])
def test_narrow_packed_row_major_b(cfg, M, N, K):
    """Row-major B stored packed (ldb = N) and ending at the end of its buffer
    region (guard sentinels, NaN, right after it): the 16-byte loads of the
    last k rows must not take values past B's last element, and columns at
    or past N must read as zero, so the exact product comes out bit for bit."""
    c = mp.mpgemm_config_info(cfg)
    fmt = "bf16" if c["in_type"] == mp.MPGEMM_IN_BF16 else "f16"
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    A, B, _ = make_inputs(M, N, K, "smallint", seed=cfg * 7 + M + N + K, dtype=dtype)
    got, gC = run_layout(A, B, None, 1.0, 0.0, 0, 0, config=cfg, lda=K, ldb=N)
    ref, _ = _ref(A, B, None, 1.0, 0.0, 0, fmt)
    assert np.array_equal(got, ref.astype(np.float32)), f"config {cfg} {M}x{N}x{K}: not bitwise"
    assert gC.untouched_outside_window()


@pytest.mark.parametrize("cfg", _narrow_ids())
def test_narrow_bias_and_scale(cfg):
    c = mp.mpgemm_config_info(cfg)
    lb = c["layout_b"]
    fmt = "bf16" if c["in_type"] == mp.MPGEMM_IN_BF16 else "f16"
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    M, N, K = 700, 11, 333
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg + 5, c_init="uniform", dtype=dtype)
    bias = np.linspace(-1.0, 1.0, N).astype(np.float32)
    got, _ = run_layout(A, B, C, 0.75, -1.25, 0, lb, config=cfg, bias=bias)
    ref, absdot = _ref(A, B, C, 0.75, -1.25, lb, fmt, bias=bias)
    assert_close(f"config {cfg} bias", got, ref, absdot, K=K, alpha=0.75, beta=-1.25, C0=C, bias=bias)


def test_narrow_entries_refuse_what_they_cannot_run():
    cfg = _narrow_ids()[0]
    dev = device()
    A = torch.zeros(64, 32, dtype=torch.float16, device=dev)
    B = torch.zeros(32, 17, dtype=torch.float16, device=dev)
    C = torch.zeros(64, 17, device=dev)
    with pytest.raises(mp.MpgemmError) as e:
        mp.gemm(A, B, C, config=cfg)             # N = 17
    assert e.value.code == mp.MPGEMM_ECONFIG
    At = torch.zeros(32, 64, dtype=torch.float16, device=dev).t()
    with pytest.raises(mp.MpgemmError) as e:
        mp.gemm(At, B[:, :16], C[:, :16], config=cfg)   # A column-major
    assert e.value.code == mp.MPGEMM_ECONFIG
