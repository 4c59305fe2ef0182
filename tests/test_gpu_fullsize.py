"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the factory's choice), element by element against the CPU
oracle, as "Capstone 4: a tensor-core GEMM" checks every element of its
products against the double-precision result (sections "Compare like with
like" and "Results").

* 2048^3 (the headline) and the tall-skinny 32768x128x4096 workload: every
  element.
* 8192^3: every element, against the oracle's library-matmul form of the
  product (the C loop would take about half an hour here); and, against the
  loop form itself, every element of whole 256x256 output tiles -- one tile
  at each of the 8 XCD slots in each of the 4 rounds of 256 workgroups the
  1024-tile grid runs in, and the four corner tiles -- plus the whole first
  and last rows and columns (an entry of every edge tile), and Freivalds'
  check over the whole output.

Each comparison also applies the accumulation diagnostic (the error against
the worst case of an FP32 running sum of K products).
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import WORKLOADS, bits, workload_inputs
from tests.gpu_util import assert_close, freivalds_ok, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["square2048", "tallskinny32768x128x4096"])
def test_workload_every_element(name):
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    got, gC = run(A, B, C, w.alpha, w.beta)
    assert gC.untouched_outside_window()
    print(f"[{name}] oracle over all {w.M * w.N} entries ({oracle.num_threads()} threads)", flush=True)
    ref, absdot = oracle.gemm(bits(A), bits(B), None if C is None else C.numpy(), w.alpha, w.beta)
    assert_close(name, got, ref, absdot, K=w.K, alpha=w.alpha, beta=w.beta, C0=C)


def test_square8192_every_element():
    w = WORKLOADS["square8192"]
    A, B, C = workload_inputs(w)
    got, gC = run(A, B, C, w.alpha, w.beta)
    assert gC.untouched_outside_window()
    print(f"[square8192] oracle (library-matmul form) over all {w.M * w.N} entries", flush=True)
    ref, absdot = oracle.gemm_matmul(bits(A), bits(B), None if C is None else C.numpy(), w.alpha, w.beta)
    assert_close("square8192", got, ref, absdot, K=w.K, alpha=w.alpha, beta=w.beta, C0=C)


def kernel_tile(bid, nb, tiles_m, tiles_n, group_m=8, xcds=8):
    """The output tile workgroup `bid` of an `nb`-workgroup grid computes:
    the kernel's tile order (consecutive ids go round-robin to the XCDs;
    each XCD takes a contiguous run of tile ids, walked in groups of
    `group_m` tile rows).  Used only to choose which tiles to check."""
    xcd, local = bid % xcds, bid // xcds
    per, rem = nb // xcds, nb % xcds
    t = xcd * (per + 1) + local if xcd < rem else rem * (per + 1) + (xcd - rem) * per + local
    group = group_m * tiles_n
    first_m = (t // group) * group_m
    gsize = min(tiles_m - first_m, group_m)
    in_group = t % group
    return first_m + in_group % gsize, in_group // gsize


def test_kernel_tile_order_is_a_permutation():
    for tm_, tn_ in ((32, 32), (16, 16), (13, 7)):
        nb = tm_ * tn_
        tiles = {kernel_tile(b, nb, tm_, tn_) for b in range(nb)}
        assert tiles == {(i, j) for i in range(tm_) for j in range(tn_)}


def test_square8192_whole_tiles_rows_and_columns():
    w = WORKLOADS["square8192"]
    A, B, _ = workload_inputs(w)
    cfg = mp.query_for(A.cuda(), B.cuda(), torch.empty(w.M, w.N, device="cuda"))
    T = cfg["bm"]
    assert (cfg["bm"], cfg["bn"]) == (256, 256) and cfg["grid"] == 1024
    got, gC = run(A, B, None, w.alpha, w.beta)
    assert np.all(np.isfinite(got)), "non-finite output"
    assert gC.untouched_outside_window()
    Ab, Bb = bits(A), bits(B)
    tiles_m, tiles_n = w.M // T, w.N // T
    nb = tiles_m * tiles_n
    rng = np.random.default_rng(w.seed)
    tiles = []
    for rnd in range(nb // 256):                  # 4 rounds of 256 resident workgroups
        for x in range(8):                        # each XCD slot
            bid = 256 * rnd + x + 8 * int(rng.integers(0, 32))
            tiles.append(kernel_tile(bid, nb, tiles_m, tiles_n))
    tiles += [(0, 0), (0, tiles_n - 1), (tiles_m - 1, 0), (tiles_m - 1, tiles_n - 1)]
    tiles = sorted(set(tiles))
    print(f"[square8192] {len(tiles)} whole tiles: {tiles}", flush=True)
    for i, (tm, tn) in enumerate(tiles):
        r0, c0 = tm * T, tn * T
        ref, absdot = oracle.gemm(Ab[r0:r0 + T], Bb[:, c0:c0 + T], None, w.alpha, w.beta)
        assert_close(f"square8192 tile ({tm},{tn})", got[r0:r0 + T, c0:c0 + T], ref, absdot, K=w.K,
                     alpha=w.alpha)
    # the first and last rows and columns, whole
    rows = np.concatenate([np.zeros(w.N), np.full(w.N, w.M - 1), np.arange(w.M), np.arange(w.M)]).astype(np.int64)
    cols = np.concatenate([np.arange(w.N), np.arange(w.N), np.zeros(w.M), np.full(w.M, w.N - 1)]).astype(np.int64)
    ref, absdot = oracle.gemm_entries(Ab, Bb, None, w.alpha, w.beta, rows, cols)
    assert_close("square8192 edge rows/columns", got[rows, cols], ref, absdot, rows, cols, K=w.K, alpha=w.alpha)
    ok, ratio = freivalds_ok(got, A, B, None, w.alpha, w.beta, seed=w.seed)
    print(f"[square8192] Freivalds worst ratio {ratio:.3g}", flush=True)
    assert ok, f"Freivalds check failed (worst err/bound {ratio:.3g})"
