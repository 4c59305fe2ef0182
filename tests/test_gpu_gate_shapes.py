"""GPU parity on the gate shapes of "Capstone 4: a tensor-core GEMM"
(section "Independent gate"): a single 16x16x16 tile, a 16x8x16 fragment,
128^3, the odd 611x613x617 case, the skinny 4096x16x4096 case, 1024^3 with
normal inputs, 256^3 with adversarial FP16 edge values (+-65504, subnormals,
the smallest normal, zeros, mixed signs; no FP32 overflow possible), and the
4096^3 timing shape.  Every element against the oracle where the oracle
finishes in seconds; sampled entries (one in every 128x128 block, the last
row and column, the corners) plus Freivalds' whole-output check at 4096^3.
Each shape runs with beta = 0 on a NaN-poisoned C and with alpha = 1.5,
beta = 0.5 on a prefilled C.
"""
import numpy as np
import pytest

import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, freivalds_ok, run, tile_samples

pytestmark = pytest.mark.gpu

FULL = [("unit", 16, 16, 16, "uniform"), ("onefrag", 16, 8, 16, "uniform"), ("cube128", 128, 128, 128, "uniform"),
        ("odd", 611, 613, 617, "uniform"), ("skinny", 4096, 16, 4096, "uniform"),
        ("normal1024", 1024, 1024, 1024, "normal4"), ("adversarial256", 256, 256, 256, "adversarial")]


@pytest.mark.parametrize("name,M,N,K,dist", FULL)
def test_gate_shape_every_element(name, M, N, K, dist):
    A, B, C = make_inputs(M, N, K, dist, seed=M + 3 * N + 7 * K, c_init="uniform")
    for alpha, beta, c0 in ((1.0, 0.0, None), (1.5, 0.5, C)):
        got, gC = run(A, B, c0, alpha, beta)
        ref, absdot = oracle.gemm(bits(A), bits(B), None if c0 is None else c0.numpy(), alpha, beta)
        assert_close(f"{name} alpha={alpha} beta={beta}", got, ref, absdot, K=K, alpha=alpha)
        assert gC.untouched_outside_window()


def test_gate_shape_4096_sampled_and_freivalds():
    M = N = K = 4096
    A, B, C = make_inputs(M, N, K, "uniform", seed=4096, c_init="uniform")
    rows, cols = tile_samples(M, N, tile=128, per_tile=1, seed=4096)
    for alpha, beta, c0 in ((1.0, 0.0, None), (1.5, 0.5, C)):
        got, _ = run(A, B, c0, alpha, beta)
        assert np.all(np.isfinite(got))
        ref, absdot = oracle.gemm_entries(bits(A), bits(B), None if c0 is None else c0.numpy(), alpha, beta,
                                          rows, cols)
        assert_close(f"4096 beta={beta}", got[rows, cols], ref, absdot, rows, cols, K=K, alpha=alpha)
        ok, ratio = freivalds_ok(got, A, B, c0, alpha, beta, seed=4096)
        assert ok, f"4096 beta={beta}: Freivalds failed (worst {ratio:.3g})"
