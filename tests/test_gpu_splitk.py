"""GPU parity for split-K (products whose tile grid leaves compute units
idle, e.g. the "skinny" 4096 x 16 x 4096 case of "Capstone 4: a tensor-core
GEMM", section "Independent gate"), through mpgemm_gemm_splitk against the
CPU oracle.  The K pieces are summed in a fixed order, so results must also
be bit-identical run to run.

Acceptance: |C_gpu - C_ref| <= 1e-3 * sum_k |a_ik b_kj| + 1e-5 elementwise;
exact small integers bit for bit.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import Guarded, assert_close, device, stored

pytestmark = pytest.mark.gpu


def run_split(A, B, C0, alpha, beta, la=0, lb=0, splits=0, bias=None, ldc=None):
    M, K = A.shape
    N = B.shape[1]
    dev = device()
    Ad = stored(A, la).to(dev)
    Bd = stored(B, lb).to(dev)
    a_view = Ad.t() if la else Ad
    b_view = Bd.t() if lb else Bd
    if C0 is None:
        gC = Guarded(torch.zeros((M, N), dtype=torch.float32), ld=ldc, fill=float("nan"))
    else:
        gC = Guarded(C0, ld=ldc)
    bias_d = None if bias is None else torch.as_tensor(bias).to(dev)
    plan = mp.splitk_plan_for(a_view, b_view, gC.view(), splits)
    mp.gemm_splitk(a_view, b_view, gC.view(), alpha, beta, bias=bias_d, splits=splits)
    torch.cuda.synchronize()
    return gC.result(), gC, plan


def check(label, A, B, C0, alpha, beta, la=0, lb=0, splits=0, bias=None, ldc=None, want_split=True):
    got, gC, plan = run_split(A, B, C0, alpha, beta, la, lb, splits, bias, ldc)
    if want_split:
        assert plan["splits"] > 1, f"{label}: expected a split plan, got {plan}"
    in_type = "bf16" if A.dtype == torch.bfloat16 else "f16"
    ref, absdot = oracle.gemm(bits(stored(A, la)), bits(stored(B, lb)),
                              None if C0 is None else C0.numpy(), alpha, beta,
                              layout_a=la, layout_b=lb, in_type=in_type, bias=bias)
    assert_close(f"{label} ({plan['splits']} pieces)", got, ref, absdot, K=A.shape[1], alpha=alpha, beta=beta,
                 C0=C0, bias=bias)
    assert gC.untouched_outside_window(), f"{label}: wrote outside the M x N window"
    return got, plan


def test_skinny_case_from_the_pages():
    """4096 x 16 x 4096, symmetric uniform: the plan keeps the narrow kernel
    whole (256 row groups of 16 already fill the chip); forced pieces run the
    tiled kernel split, and both match the oracle."""
    A, B, _ = make_inputs(4096, 16, 4096, "uniform", seed=81)
    print("[splitk] skinny", flush=True)
    _, plan = check("skinny", A, B, None, 1.0, 0.0, want_split=False)
    assert plan["splits"] == 1 and mp.mpgemm_config_info(plan["config_id"])["kind_name"] == "narrow"
    _, plan = check("skinny forced", A, B, None, 1.0, 0.0, splits=16)
    assert plan["splits"] == 16 and mp.mpgemm_config_info(plan["config_id"])["kind_name"] == "pipe"


def test_short_skinny_deep_k_splits_by_itself():
    """256 x 16 x 65536: 16 row groups cannot fill the chip, so the plan
    splits K across a tiled kernel."""
    A, B, C = make_inputs(256, 16, 65536, "uniform", seed=83, c_init="uniform")
    _, plan = check("short skinny", A, B, C, 0.5, 2.0)
    assert mp.mpgemm_config_info(plan["config_id"])["kind_name"] == "pipe"


@pytest.mark.parametrize("splits", [2, 3, 5, 7, 16])
def test_forced_splits_ragged(splits):
    M, N, K = 300, 200, 1234
    A, B, C = make_inputs(M, N, K, "uniform", seed=82 + splits, c_init="uniform")
    check(f"ragged splits={splits}", A, B, C, 1.5, 0.5, splits=splits, ldc=211)


def test_more_pieces_than_k_tiles_is_capped():
    A, B, _ = make_inputs(130, 70, 100, "uniform", seed=88)
    _, plan = check("capped", A, B, None, 1.0, 0.0, splits=64)
    assert plan["splits"] <= 4


@pytest.mark.parametrize("la,lb", [(0, 1), (1, 0), (1, 1)])
def test_layouts(la, lb):
    """A ragged K past 4096 with two tiles of C: the automatic plan splits it."""
    A, B, C = make_inputs(256, 96, 5000, "uniform", seed=90 + la + 2 * lb, c_init="uniform")
    check(f"layout {la}{lb}", A, B, C, 0.75, -1.0, la, lb)


def test_floor_of_six_pieces_on_a_larger_grid():
    """512 x 768 x 4096 (96 tiles of 64 x 64): the automatic plan takes 6
    pieces of about 683 K rather than 4 of 1024 K."""
    A, B, C = make_inputs(512, 768, 4096, "uniform", seed=93, c_init="uniform")
    print("[splitk] floor of six", flush=True)
    _, plan = check("floor of six", A, B, C, 1.0, 1.0)
    assert plan["splits"] == 6


def test_bf16_with_bias():
    A, B, C = make_inputs(512, 48, 4096, "uniform", seed=95, c_init="uniform", dtype=torch.bfloat16)
    bias = np.linspace(-1, 1, 48).astype(np.float32)
    check("bf16 bias", A, B, C, 1.25, 0.5, bias=bias)


def test_exact_integers_and_determinism():
    A, B, _ = make_inputs(1000, 64, 2048, "smallint", seed=96)
    g1, _, p = run_split(A, B, None, 1.0, 0.0, splits=6)
    g2, _, _ = run_split(A, B, None, 1.0, 0.0, splits=6)
    assert p["splits"] == 6
    ints = A.numpy().astype(np.int64) @ B.numpy().astype(np.int64)
    assert np.array_equal(g1, ints.astype(np.float32))
    A, B, _ = make_inputs(1000, 64, 2048, "uniform", seed=97)
    g1, _, _ = run_split(A, B, None, 1.0, 0.0, splits=5)
    g2, _, _ = run_split(A, B, None, 1.0, 0.0, splits=5)
    assert np.array_equal(g1, g2)


@pytest.mark.parametrize("splits", [2, 3])
def test_forced_splits_on_the_staggered_k_order_entry(splits):
    """Forced pieces on a shape the 128x128x128 entry takes: its workgroups
    walk their piece's K tiles in a rotated order (k_order 2), so every
    piece's K range must still be covered once.  Exact small integers make
    every order give the same bits; uniform inputs go to the oracle."""
    M, N, K = 1024, 2048, 1024 + 640
    A, B, _ = make_inputs(M, N, K, "smallint", seed=98)
    got, _, plan = run_split(A, B, None, 1.0, 0.0, splits=splits)
    c = mp.mpgemm_config_info(plan["config_id"])
    assert plan["splits"] == splits and (c["bm"], c["bn"], c["bk"], c["k_order"]) == (128, 128, 128, 2), plan
    # small integers: every product and sum is exact in float64 as in FP32
    exact = A.numpy().astype(np.float64) @ B.numpy().astype(np.float64)
    assert np.array_equal(got, exact.astype(np.float32))
    A, B, C = make_inputs(M, N, K, "uniform", seed=99, c_init="uniform")
    check(f"staggered splits={splits}", A, B, C, 1.5, 0.5, splits=splits)


def test_single_piece_is_the_ordinary_path():
    """A full grid plans one piece and needs no workspace: bit for bit the
    ordinary call."""
    A, B, _ = make_inputs(2048, 2048, 512, "uniform", seed=98)
    got, _, plan = run_split(A, B, None, 1.0, 0.0)
    assert plan["splits"] == 1 and plan["workspace_bytes"] == 0
    dev = device()
    C = torch.empty(2048, 2048, device=dev)
    mp.gemm(A.to(dev), B.to(dev), C)
    torch.cuda.synchronize()
    assert np.array_equal(got, C.cpu().numpy())


def test_workspace_errors_on_the_device_path():
    dev = device()
    A = torch.zeros(256, 65536, dtype=torch.float16, device=dev)
    B = torch.zeros(65536, 16, dtype=torch.float16, device=dev)
    C = torch.zeros(256, 16, device=dev)
    small = torch.empty(16, device=dev)
    with pytest.raises(mp.MpgemmError) as e:
        mp.gemm_splitk(A, B, C, workspace=small)
    assert e.value.code == mp.MPGEMM_EWORKSPACE
