"""GPU: mpgemm_gemm_splitk_static, split-K whose partial products go to the
library's static device scratch (no allocation, for callers that cannot
allocate), called through the C ABI and checked against
mpgemm_gemm_splitk with a caller-provided workspace -- the same plan and
kernels, so bit for bit -- and against the oracle within the acceptance
rule.  Two calls in a row, the second smaller (the scratch keeps the first
call's partials and must not leak into the second); a plan larger than the
scratch is refused before anything is enqueued; a one-piece plan is the
ordinary path.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, device

pytestmark = pytest.mark.gpu


def _calls(A, B, C0, alpha, beta, splits, bias=None):
    """(result of the static-scratch call, result of the workspace call, plan)
    on the same inputs; C starts as C0 or NaN (beta == 0)."""
    dev = device()
    M, K = A.shape
    N = B.shape[1]
    Ad, Bd = A.to(dev), B.to(dev)
    bias_d = None if bias is None else torch.as_tensor(bias).to(dev)
    bias_ptr = 0 if bias_d is None else bias_d.data_ptr()
    args = (mp.MPGEMM_IN_F16, 0, 0, M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N)
    plan = mp.mpgemm_splitk_plan(*args, splits)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for static in (True, False):
        Cd = (C0.clone() if C0 is not None else torch.full((M, N), float("nan"))).to(dev)
        if static:
            rc = mp.mpgemm_gemm_splitk_static(*args, Cd.data_ptr(), N, alpha, beta, bias_ptr, splits, stream)
        else:
            ws = torch.empty(max(plan["workspace_bytes"] // 4, 1), dtype=torch.float32, device=dev)
            rc = mp.mpgemm_gemm_splitk(*args, Cd.data_ptr(), N, alpha, beta, bias_ptr, splits, ws.data_ptr(),
                                       ws.numel() * 4, stream)
        assert rc == mp.MPGEMM_OK, mp.mpgemm_strerror(rc)
        torch.cuda.synchronize()
        outs.append(Cd.cpu().numpy())
    return outs[0], outs[1], plan


def test_static_scratch_equals_the_workspace_entry_point_on_two_calls():
    # first call: 256 x 16 x 65536, the automatic plan (many pieces)
    A, B, C = make_inputs(256, 16, 65536, "uniform", seed=301, c_init="uniform")
    st, ws, plan = _calls(A, B, C, 1.5, 0.5, 0)
    print(f"[static scratch] first call: {plan}", flush=True)
    assert plan["splits"] > 1 and plan["workspace_bytes"] <= mp.MPGEMM_STATIC_SCRATCH_BYTES
    assert np.array_equal(st, ws), "static scratch differs from the workspace entry point"
    ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5)
    assert_close("static scratch, first call", st, ref, absdot, K=65536, alpha=1.5, beta=0.5, C0=C)
    # second call, smaller, with a bias and beta == 0 (C NaN-poisoned)
    A, B, _ = make_inputs(100, 48, 8192, "uniform", seed=302)
    bias = np.linspace(-1, 1, 48).astype(np.float32)
    st, ws, plan = _calls(A, B, None, 1.0, 0.0, 6, bias=bias)
    print(f"[static scratch] second call: {plan}", flush=True)
    assert plan["splits"] == 6
    assert np.array_equal(st, ws), "static scratch differs from the workspace entry point"
    ref, absdot = oracle.gemm(bits(A), bits(B), None, 1.0, 0.0, bias=bias)
    assert_close("static scratch, second call", st, ref, absdot, K=8192, alpha=1.0, bias=bias)


def test_static_scratch_refuses_a_plan_larger_than_itself():
    dev = device()
    M = N = 2048
    K = 8192
    A = torch.zeros(M, K, dtype=torch.float16, device=dev)
    B = torch.zeros(K, N, dtype=torch.float16, device=dev)
    C = torch.full((M, N), float("nan"), device=dev)
    plan = mp.mpgemm_splitk_plan(mp.MPGEMM_IN_F16, 0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N, 4)
    assert plan["workspace_bytes"] > mp.MPGEMM_STATIC_SCRATCH_BYTES
    rc = mp.mpgemm_gemm_splitk_static(mp.MPGEMM_IN_F16, 0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                      C.data_ptr(), N, 1.0, 0.0, 0, 4, torch.cuda.current_stream().cuda_stream)
    assert rc == mp.MPGEMM_ESCRATCH
    torch.cuda.synchronize()
    assert bool(torch.isnan(C).all()), "a refused call wrote C"


def test_single_piece_plan_is_the_ordinary_path():
    A, B, _ = make_inputs(1024, 1024, 512, "uniform", seed=303)
    st, ws, plan = _calls(A, B, None, 1.0, 0.0, 0)
    assert plan["splits"] == 1 and plan["workspace_bytes"] == 0
    assert np.array_equal(st, ws)
