"""GPU parity of the factory's measured rules, each on a product that the
rule decides, in the launch configuration the factory picks (asserted from
the query): every element against the oracle's C loop, or whole row blocks
where the product is large.

* short K over many tiles: 64x64x64 tiles (3072x3072x128);
* one 128-column band: 128x128x128 tiles up to K = 1024 (32768x128x1024);
* row-major FP16 whose B rows are not 16-byte aligned, with a sparse second
  round of 128x128 tiles: 64x64x128 tiles (2049x2049x2048);
* A row-major with B column-major: 256x256 tiles at 2.5 times their rounds
  (1504x12052x2229; the first, a middle and the last 32 rows).
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, run, run_layout, stored

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K,shape", [
    (3072, 3072, 128, (64, 64, 64)),
    (32768, 128, 1024, (128, 128, 128)),
    (2049, 2049, 2048, (64, 64, 128)),
])
def test_factory_rule_every_element(M, N, K, shape):
    print(f"[factory rule] {M}x{N}x{K}", flush=True)
    A, B, C = make_inputs(M, N, K, "uniform", seed=M * 7 + N * 3 + K, c_init="uniform")
    cfg = mp.mpgemm_f16f32_query(M, N, K, 0x7F0000000000, K, 0x7F1000000000, N, 0x7F2000000000, N, 1.25, 0.5)
    assert (cfg["bm"], cfg["bn"], cfg["bk"]) == shape, cfg
    got, gC = run(A, B, C, 1.25, 0.5)
    assert gC.untouched_outside_window()
    ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 1.25, 0.5)
    assert_close(f"{M}x{N}x{K}", got, ref, absdot, K=K, alpha=1.25, beta=0.5, C0=C)
    torch.cuda.empty_cache()


def test_factory_big_tile_for_b_column_major_row_blocks():
    M, N, K = 1504, 12052, 2229
    print(f"[factory rule] {M}x{N}x{K} A row-major, B column-major", flush=True)
    A, B, _ = make_inputs(M, N, K, "uniform", seed=4242)
    cfg = mp.mpgemm_f16f32_layout_query(0, 1, M, N, K, 0x7F0000000000, K, 0x7F1000000000, K,
                                        0x7F2000000000, N, 1.0, 0.0)
    assert cfg["bm"] == 256 and cfg["layout_b"] == 1, cfg
    got, gC = run_layout(A, B, None, 1.0, 0.0, 0, 1)
    assert gC.untouched_outside_window()
    rows = np.r_[0:32, M // 2 - 16:M // 2 + 16, M - 32:M]
    ref, absdot = oracle.gemm(bits(A[rows]), bits(B), None, 1.0, 0.0)
    assert_close("1504x12052x2229 rows", got[rows], ref, absdot, K=K, alpha=1.0)
    torch.cuda.empty_cache()
