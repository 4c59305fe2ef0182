"""NaN and Inf inputs (the pages are silent; IEEE semantics decide): the GPU's
pattern of NaN, +Inf and -Inf outputs must equal the oracle's exactly (NaN
times anything is NaN, 0 * Inf is NaN, Inf - Inf is NaN; finite FP16
products cannot overflow the FP32 sum at these sizes), and every finite
output must meet the tolerance.  Every pipelined config, in its storage
order and input format, on a ragged shape with a NaN inside the K tail (the
last K % 8 values, which go through their own matrix-instruction step), an
+Inf inside the matrix, a -Inf in the last column, and a zero that meets
that -Inf.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import run_layout, stored

pytestmark = pytest.mark.gpu


def _pipe_ids():
    return [i for i in range(mp.mpgemm_num_configs()) if mp.mpgemm_config_info(i)["kind_name"] == "pipe"]


@pytest.mark.parametrize("cfg", _pipe_ids())
def test_nonfinite_pattern_matches_the_oracle(cfg):
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    bf16 = c["in_type"] == mp.MPGEMM_IN_BF16
    dtype = torch.bfloat16 if bf16 else torch.float16
    M, N, K = 261, 147, 101
    A, B, _ = make_inputs(M, N, K, "uniform", seed=cfg + 900, dtype=dtype)
    A, B = A.clone(), B.clone()
    A[5, 100] = float("nan")       # in the K tail: row 5 all NaN
    A[130, 3] = float("inf")       # row 130: +-Inf (NaN where B[3, j] == 0 or meets -Inf)
    B[3, 7] = 0.0                  # Inf * 0 = NaN at (130, 7)
    B[50, N - 1] = float("-inf")   # last column: -+Inf
    A[M - 1, 50] = 0.0             # 0 * -Inf = NaN at (M-1, N-1)
    got, gC = run_layout(A, B, None, 1.0, 0.0, la, lb, config=cfg)
    ref, absdot = oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)), None, 1.0, 0.0, layout_a=la,
                              layout_b=lb, in_type="bf16" if bf16 else "f16")
    label = f"config {cfg}"
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{label}: NaN pattern differs"
    assert np.array_equal(np.isposinf(got), np.isposinf(ref)), f"{label}: +Inf pattern differs"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{label}: -Inf pattern differs"
    assert np.isnan(ref[5]).all() and np.isnan(ref[130, 7]) and np.isnan(ref[M - 1, N - 1])
    fin = np.isfinite(ref)
    assert oracle.tolerance_ok(got[fin], ref[fin], absdot[fin]).all(), f"{label}: finite entries out of tolerance"
    assert oracle.accumulation_ratio(got[fin], ref[fin], absdot[fin], K, 1.0) <= 1.0
    assert gC.untouched_outside_window()
