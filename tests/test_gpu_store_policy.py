"""GPU parity of both cache policies of the 256x256 kernels' C stores
(non-temporal, plain), which the host picks per call: every element against
the oracle's C loop, the guard margins and the ld gap of C untouched, and
the policy the query reports checked against the one the case is built to
take.

* nearly a full round of 256x256 tiles at short K, C rows 128-byte
  aligned: plain;
* the same with at most 176 tiles: non-temporal;
* C rows that start mid-line (odd N, so ldc is odd): plain;
* alpha/beta with a C read, plain and non-temporal.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import Guarded, assert_close, device

pytestmark = pytest.mark.gpu


def _run(M, N, K, alpha, beta, ldc, seed):
    A, B, C0 = make_inputs(M, N, K, "uniform", seed=seed, c_init="uniform" if beta != 0.0 else None)
    gA, gB = Guarded(A), Guarded(B)
    gC = Guarded(C0 if C0 is not None else torch.zeros((M, N)), ld=ldc,
                 fill=None if C0 is not None else float("nan"))
    # the C window starts GUARD elements into a fresh allocation: 128-byte
    # aligned when GUARD * 4 is a multiple of 128
    Cv = gC.view()
    cfg = mp.query_for(gA.view(), gB.view(), Cv, alpha, beta)
    mp.gemm(gA.view(), gB.view(), Cv, alpha, beta)
    torch.cuda.synchronize()
    got = gC.result()
    assert gC.untouched_outside_window()
    ref, absdot = oracle.gemm(bits(A), bits(B), None if C0 is None else C0.numpy(), alpha, beta)
    return cfg, got, ref, absdot, C0


@pytest.mark.parametrize("M,N,K,ldc,alpha,beta,stores", [
    (3584, 4096, 384, None, 1.0, 0.0, 0),       # 224 tiles, one round, K < 2048: plain
    (3584, 4096, 320, None, 1.5, 0.5, 0),       # ... with the C read
    (3328, 3328, 384, None, 1.0, 0.0, 1),       # 169 tiles: non-temporal
    (2816, 3072, 512, None, -0.75, 2.0, 1),     # 132 tiles, with the C read
    (1457, 10609, 128, None, 1.0, 0.0, 0),      # odd ldc: rows start mid-line, plain
    (3328, 3328, 300, 3333, 1.0, 0.5, 0),       # odd ldc and a K tail
])
def test_big_tile_store_policies(M, N, K, ldc, alpha, beta, stores):
    print(f"[store policy] {M}x{N}x{K} ldc={ldc} alpha={alpha} beta={beta}", flush=True)
    cfg, got, ref, absdot, C0 = _run(M, N, K, alpha, beta, ldc, seed=M + N + K)
    assert cfg["bm"] == 256, cfg
    assert cfg["c_stores"] == stores, cfg
    assert np.isfinite(got).all()
    assert_close(f"{M}x{N}x{K} stores={stores}", got, ref, absdot, K=K, alpha=alpha, beta=beta, C0=C0)
    torch.cuda.empty_cache()
