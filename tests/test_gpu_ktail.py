"""GPU parity of the K tail (the zero-fill repair of a K that no tile divides,
"Capstone 4: a tensor-core GEMM", Practice 3).

When K % 8 != 0 the pipelined kernels run their LDS copy loop over the largest
multiple of 8 of K and add the last K % 8 values as one more matrix
instruction step whose operands are loaded straight from memory, zero past the
edge.  Every pipelined config, in its storage order and input format, runs K
values that leave the tail alone (K < 8), a tail after one partial K tile,
and a tail after several whole K tiles.  Each stored operand is padded past
its rows (leading dimension > extent) and guarded, and the padding and guards
hold a NaN pattern, so a read past the K (or M/N) edge that is not zeroed
turns the result into NaN.  Small integers make every sum exact, so the
result must equal the oracle's bit for bit; uniform inputs with beta != 0
are checked against the tolerance.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, run_layout, stored

pytestmark = pytest.mark.gpu


def _pipe_ids():
    return [i for i in range(mp.mpgemm_num_configs()) if mp.mpgemm_config_info(i)["kind_name"] == "pipe"]


def _ref(A, B, C0, alpha, beta, la, lb, in_type):
    return oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)), None if C0 is None else C0.numpy(),
                       alpha, beta, layout_a=la, layout_b=lb, in_type=in_type)


@pytest.mark.parametrize("K", [5, 13, 263])
@pytest.mark.parametrize("cfg", _pipe_ids())
def test_k_tail_every_pipe_config(cfg, K):
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    bf16 = c["in_type"] == mp.MPGEMM_IN_BF16
    dtype = torch.bfloat16 if bf16 else torch.float16
    in_type = "bf16" if bf16 else "f16"
    M, N = 97, 75
    # stored rows: A (M,K) or (K,M), B (K,N) or (N,K); pad each by a few elements
    lda = (M if la else K) + 3
    ldb = (K if lb else N) + 5
    A, B, _ = make_inputs(M, N, K, "smallint", seed=cfg * 31 + K, dtype=dtype)
    got, gC = run_layout(A, B, None, 1.0, 0.0, la, lb, config=cfg, lda=lda, ldb=ldb)
    ref, _ = _ref(A, B, None, 1.0, 0.0, la, lb, in_type)
    assert np.array_equal(got, ref.astype(np.float32)), \
        f"config {cfg} K={K}: not bitwise (max diff {np.nanmax(np.abs(got - ref)):.3g}, NaN {np.isnan(got).sum()})"
    assert gC.untouched_outside_window()
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg * 37 + K, c_init="uniform", dtype=dtype)
    got, gC = run_layout(A, B, C, 1.5, 0.5, la, lb, config=cfg, lda=lda, ldb=ldb, ldc=N + 2)
    ref, absdot = _ref(A, B, C, 1.5, 0.5, la, lb, in_type)
    assert_close(f"config {cfg} K={K} beta=.5", got, ref, absdot, K=K, alpha=1.5, beta=0.5, C0=C)
    assert gC.untouched_outside_window()
