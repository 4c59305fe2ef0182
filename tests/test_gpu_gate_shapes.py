"""GPU parity on the gate shapes of "Capstone 4: a tensor-core GEMM"
(section "Independent gate"): a single 16x16x16 tile, a 16x8x16 fragment,
128^3, the odd 611x613x617 case, the skinny 4096x16x4096 case, 1024^3 with
normal inputs, 256^3 with adversarial FP16 edge values (+-65504, subnormals,
the smallest normal, zeros, mixed signs; no FP32 overflow possible), and the
4096^3 timing shape.  Every element against the oracle; at 4096^3 against
its library-matmul form, and, against the C loop itself, every element of
eight whole 256x256 output tiles (the corners and four more) and of the
first and last rows and columns, plus Freivalds' whole-output check.
Each shape runs with beta = 0 on a NaN-poisoned C and with alpha = 1.5,
beta = 0.5 on a prefilled C.
"""
import numpy as np
import pytest

import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, freivalds_ok, run

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
        assert_close(f"{name} alpha={alpha} beta={beta}", got, ref, absdot, K=K, alpha=alpha, beta=beta, C0=c0)
        assert gC.untouched_outside_window()


def test_gate_shape_4096_tiles_edges_and_freivalds():
    M = N = K = 4096
    T = 256
    A, B, C = make_inputs(M, N, K, "uniform", seed=4096, c_init="uniform")
    Ab, Bb = bits(A), bits(B)
    rng = np.random.default_rng(4096)
    tiles = {(0, 0), (0, N // T - 1), (M // T - 1, 0), (M // T - 1, N // T - 1)}
    while len(tiles) < 8:
        tiles.add((int(rng.integers(0, M // T)), int(rng.integers(0, N // T))))
    edge_rows = np.concatenate([np.zeros(N), np.full(N, M - 1), np.arange(M), np.arange(M)]).astype(np.int64)
    edge_cols = np.concatenate([np.arange(N), np.arange(N), np.zeros(M), np.full(M, N - 1)]).astype(np.int64)
    for alpha, beta, c0 in ((1.0, 0.0, None), (1.5, 0.5, C)):
        got, _ = run(A, B, c0, alpha, beta)
        assert np.all(np.isfinite(got))
        cn = None if c0 is None else c0.numpy()
        ref, absdot = oracle.gemm_matmul(Ab, Bb, cn, alpha, beta)
        assert_close(f"4096 beta={beta} every element", got, ref, absdot, K=K, alpha=alpha, beta=beta, C0=cn)
        for tm, tn in sorted(tiles):
            r0, c0_ = tm * T, tn * T
            ref, absdot = oracle.gemm(Ab[r0:r0 + T], Bb[:, c0_:c0_ + T],
                                      None if cn is None else np.ascontiguousarray(cn[r0:r0 + T, c0_:c0_ + T]),
                                      alpha, beta)
            assert_close(f"4096 beta={beta} tile ({tm},{tn})", got[r0:r0 + T, c0_:c0_ + T], ref, absdot,
                         K=K, alpha=alpha, beta=beta, C0=None if cn is None else cn[r0:r0 + T, c0_:c0_ + T])
        ref, absdot = oracle.gemm_entries(Ab, Bb, cn, alpha, beta, edge_rows, edge_cols)
        assert_close(f"4096 beta={beta} edge rows/columns", got[edge_rows, edge_cols], ref, absdot, edge_rows,
                     edge_cols, K=K, alpha=alpha, beta=beta, C0=cn)
        ok, ratio = freivalds_ok(got, A, B, c0, alpha, beta, seed=4096)
        assert ok, f"4096 beta={beta}: Freivalds failed (worst {ratio:.3g})"
