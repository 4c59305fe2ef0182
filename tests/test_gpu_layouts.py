"""GPU parity for A and/or B stored column-major (the operand layout of
"Capstone 4: a tensor-core GEMM", Independent gate: A row-major, B
column-major), called through the C ABI's layout entry points and checked
against the CPU oracle's layout-aware product on the same stored arrays.

Acceptance as everywhere: |C_gpu - C_ref| <= 1e-3 * sum_k |a_ik b_kj| + 1e-5
elementwise; exact small-integer inputs must match bit for bit.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import (assert_close, freivalds_ok, run_layout, stored)

pytestmark = pytest.mark.gpu

LAYOUTS = [(0, 1), (1, 0), (1, 1)]


def oracle_layout(A, B, C0, alpha, beta, la, lb):
    return oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)),
                       None if C0 is None else C0.numpy(), alpha, beta, layout_a=la, layout_b=lb)


def full_check(label, A, B, C0, alpha, beta, la, lb, **kw):
    got, gC = run_layout(A, B, C0, alpha, beta, la, lb, **kw)
    ref, absdot = oracle_layout(A, B, C0, alpha, beta, la, lb)
    assert_close(label, got, ref, absdot, K=A.shape[1], alpha=alpha, beta=beta, C0=C0)
    assert gC.untouched_outside_window(), f"{label}: wrote outside the M x N window"
    return got


def _layout_ids():
    out = []
    for i in range(mp.mpgemm_num_configs()):
        c = mp.mpgemm_config_info(i)
        if (c["kind_name"] == "pipe" and (c["layout_a"], c["layout_b"]) != (0, 0)
                and c["in_type"] == mp.MPGEMM_IN_F16):
            out.append(i)
    return out


SHAPES = [(1, 1, 1), (15, 17, 16), (17, 15, 33), (65, 63, 129), (129, 127, 257), (611, 613, 617),
          (256, 256, 1), (300, 17, 40), (17, 300, 40), (4096, 16, 256), (16, 4096, 256)]


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_factory_edge_shapes(la, lb, M, N, K):
    A, B, C = make_inputs(M, N, K, "uniform", seed=M * 7 + N * 3 + K + la + 2 * lb, c_init="uniform")
    print(f"[{la}{lb}] {M}x{N}x{K}", flush=True)
    full_check(f"{la}{lb} {M}x{N}x{K} beta=0", A, B, None, 1.0, 0.0, la, lb)
    full_check(f"{la}{lb} {M}x{N}x{K} beta=.5", A, B, C, 1.5, 0.5, la, lb)


@pytest.mark.parametrize("cfg", _layout_ids())
def test_every_layout_config_ragged_strided(cfg):
    """M, N, K fit no tile; leading dimensions are multiples of 8 beyond the
    stored row lengths (so the 16-byte entries apply) while the extents leave
    partial vectors at the edges; ldc > N."""
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    M, N, K = 261, 147, 101
    lda = 272 if la else 112
    ldb = 112 if lb else 160
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg + 300, c_init="uniform")
    print(f"[config {cfg}] layout {la}{lb}", flush=True)
    full_check(f"config {cfg}", A, B, C, 1.25, -0.75, la, lb, config=cfg, lda=lda, ldb=ldb, ldc=151)
    full_check(f"config {cfg} beta=0", A, B, None, 1.0, 0.0, la, lb, config=cfg, lda=lda, ldb=ldb,
               ldc=149)


@pytest.mark.parametrize("cfg", _layout_ids())
def test_every_layout_config_multi_tile_bitwise(cfg):
    c = mp.mpgemm_config_info(cfg)
    la, lb = c["layout_a"], c["layout_b"]
    M, N, K = 520, 600, 392
    A, B, _ = make_inputs(M, N, K, "smallint", seed=cfg + 400)
    got, _ = run_layout(A, B, None, 1.0, 0.0, la, lb, config=cfg)
    ref, _ = oracle_layout(A, B, None, 1.0, 0.0, la, lb)
    assert np.array_equal(got, ref.astype(np.float32)), f"config {cfg}: not bitwise"


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_misaligned_and_odd_leading_dimensions(la, lb):
    M, N, K = 333, 250, 617
    A, B, C = make_inputs(M, N, K, "uniform", seed=41 + la + 2 * lb, c_init="uniform")
    a_len = M if la else K
    b_len = K if lb else N
    for a_off, b_off, lda, ldb in [(1, 0, a_len, b_len), (0, 1, a_len + 3, b_len),
                                   (1, 1, a_len + 3, b_len + 5), (0, 0, a_len, b_len + 1)]:
        q = mp.query_for(*(t.cuda() for t in (stored(A, la).t() if la else A,
                                                  stored(B, lb).t() if lb else B)),
                         torch.empty(M, N, device="cuda"))
        assert (q["layout_a"], q["layout_b"]) == (la, lb)
        full_check(f"{la}{lb} a_off={a_off} b_off={b_off} lda={lda} ldb={ldb}", A, B, C, 1.5, 0.5,
                   la, lb, a_off=a_off, b_off=b_off, lda=lda, ldb=ldb)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_direct_kernel_any_layout(la, lb):
    M, N, K = 97, 70, 45
    A, B, C = make_inputs(M, N, K, "uniform", seed=51 + la + 2 * lb, c_init="uniform")
    direct = [i for i in range(mp.mpgemm_num_configs())
              if mp.mpgemm_config_info(i)["kind_name"] == "direct"
              and mp.mpgemm_config_info(i)["in_type"] == mp.MPGEMM_IN_F16]
    full_check(f"direct {la}{lb}", A, B, C, 0.5, 1.5, la, lb, config=direct[0])


def test_same_tile_shape_is_bitwise_identical_across_layouts():
    """The storage order changes only where each operand value is fetched
    from: every MFMA sees the same operands in the same k order, so the four
    eight-wave 256x256x64 entries must agree bit for bit."""
    ids = {}
    for i in range(mp.mpgemm_num_configs()):
        c = mp.mpgemm_config_info(i)
        if (c["kind_name"], c["bm"], c["bn"], c["bk"], c["waves_m"], c["waves_n"], c["stages"],
                c["vec_a"], c["vec_b"], c["in_type"]) == ("pipe", 256, 256, 64, 2, 4, 2, 8, 8, 0):
            ids[(c["layout_a"], c["layout_b"])] = i
    assert set(ids) == {(0, 0), (0, 1), (1, 0), (1, 1)}
    M, N, K = 300, 520, 333
    A, B, C = make_inputs(M, N, K, "uniform", seed=61, c_init="uniform")
    # leading dimensions padded to multiples of 8 so the 16-byte entries apply
    lds = {0: (336, 520), 1: (304, 336)}
    outs = {lay: run_layout(A, B, C, 1.5, 0.5, *lay, config=i,
                            lda=lds[lay[0]][0] if lay[0] == 0 else lds[1][0],
                            ldb=lds[0][1] if lay[1] == 0 else lds[1][1])[0]
            for lay, i in ids.items()}
    for lay, out in outs.items():
        assert np.array_equal(out, outs[(0, 0)]), f"layout {lay} differs from row-major"


@pytest.mark.parametrize("la,lb", [(1, 0), (0, 1), (1, 1)])
def test_2048_every_element_and_freivalds(la, lb):
    M = N = K = 2048
    A, B, _ = make_inputs(M, N, K, "uniform", seed=1001 + la + 2 * lb)
    got, gC = run_layout(A, B, None, 1.0, 0.0, la, lb)
    assert np.all(np.isfinite(got))
    ref, absdot = oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)), None, 1.0, 0.0, layout_a=la, layout_b=lb)
    assert_close(f"2048 {la}{lb}", got, ref, absdot, K=K, alpha=1.0)
    ok, ratio = freivalds_ok(got, A, B, None, 1.0, 0.0, seed=5)
    assert ok, f"Freivalds failed (worst {ratio:.3g})"
