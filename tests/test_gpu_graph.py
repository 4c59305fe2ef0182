"""GPU: the library's launches recorded into a HIP graph and replayed.

The library enqueues kernels only (no memset, allocation or synchronization),
so a caller may capture its calls.  Each graph is replayed several times with
eager work of the program in between, and every replay must match the eager
call bit for bit; one case is also checked against the CPU oracle.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, device

pytestmark = pytest.mark.gpu


def _replays_match(fn, out, eager, replays=4):
    """Capture fn() (which writes `out`) into a graph; replay it `replays`
    times, with unrelated eager work and a poisoned output in between, and
    compare every replay with `eager` bit for bit."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    other = torch.randn(512, 512, device=out.device)
    for r in range(replays):
        out.fill_(float("nan"))
        other = other @ other.t() / 512.0          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {r} differs"


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (1000, 800, 617), (2048, 2048, 256)])
def test_graph_replay_equals_eager(M, N, K):
    dev = device()
    A, B, _ = make_inputs(M, N, K, "uniform", seed=M + N + K)
    Ad, Bd = A.to(dev), B.to(dev)
    C = torch.full((M, N), float("nan"), device=dev)
    mp.gemm(Ad, Bd, C, 1.5, 0.0)
    torch.cuda.synchronize()
    eager = C.clone()
    if M == 256:
        ref, absdot = oracle.gemm(bits(A), bits(B), None, 1.5, 0.0)
        assert_close("graph 256", eager.cpu().numpy(), ref, absdot, K=K, alpha=1.5)
    print(f"[graph] {M}x{N}x{K}", flush=True)
    _replays_match(lambda: mp.gemm(Ad, Bd, C, 1.5, 0.0), C, eager)


def test_graph_replay_split_k_and_bias():
    """Two kernels per call (pieces, then the ordered reduction) and a bias."""
    dev = device()
    M, N, K = 4096, 16, 4096
    A, B, _ = make_inputs(M, N, K, "uniform", seed=91)
    Ad, Bd = A.to(dev), B.to(dev)
    bias = torch.linspace(-1, 1, N, device=dev)
    C = torch.full((M, N), float("nan"), device=dev)
    plan = mp.splitk_plan_for(Ad, Bd, C, 8)
    assert plan["splits"] == 8
    ws = torch.empty(plan["workspace_bytes"] // 4, device=dev)
    mp.gemm_splitk(Ad, Bd, C, 1.0, 0.0, bias=bias, workspace=ws, splits=8)
    torch.cuda.synchronize()
    eager = C.clone()
    ref, absdot = oracle.gemm(bits(A), bits(B), None, 1.0, 0.0, bias=bias.cpu().numpy())
    assert_close("graph split-K", eager.cpu().numpy(), ref, absdot, K=K, alpha=1.0, bias=bias.cpu().numpy())
    print(f"[graph] split-K {plan['splits']} pieces", flush=True)
    _replays_match(lambda: mp.gemm_splitk(Ad, Bd, C, 1.0, 0.0, bias=bias, workspace=ws, splits=8), C, eager)
    assert np.isfinite(C.cpu().numpy()).all()
