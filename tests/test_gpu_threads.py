"""Concurrent calls: the library keeps no per-call state, so host threads may
call it at once, each on its own stream (mpgemm.h, "Ownership and
concurrency").  Five threads, each with its own stream, buffers and shapes
(different kernel configs, ragged edges, beta != 0, column-major B, BF16,
split-K, the narrow kernel), call the library repeatedly at the same time; every result must
equal the same call made alone, bit for bit (each call is deterministic)."""
import threading

import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
from dense_mixed_precision_amd.workloads import make_inputs
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

CASES = [
    dict(M=1000, N=800, K=617, dtype=torch.float16, col_b=False, splitk=False, beta=0.5),
    dict(M=2048, N=1024, K=512, dtype=torch.float16, col_b=True, splitk=False, beta=0.0),
    dict(M=513, N=257, K=1031, dtype=torch.bfloat16, col_b=False, splitk=False, beta=-1.0),
    dict(M=256, N=16, K=65536, dtype=torch.float16, col_b=False, splitk=True, beta=0.0),
    dict(M=4096, N=16, K=4096, dtype=torch.float16, col_b=False, splitk=False, beta=0.5),   # narrow
]


def _prepare(case, seed):
    A, B, C = make_inputs(case["M"], case["N"], case["K"], "uniform", seed=seed, c_init="uniform",
                          dtype=case["dtype"])
    dev = device()
    Ad = A.to(dev)
    Bd = B.t().contiguous().to(dev).t() if case["col_b"] else B.to(dev)
    return Ad, Bd, C.to(dev)


def _call(case, Ad, Bd, C0, stream, ws):
    # C0 is never written after setup, so any stream may read it; the copy
    # and the call both go on `stream`, in that order
    with torch.cuda.stream(stream):
        C = C0.clone()
        if case["splitk"]:
            mp.gemm_splitk(Ad, Bd, C, 1.0, case["beta"], workspace=ws, stream=stream)
        else:
            mp.gemm(Ad, Bd, C, 1.25, case["beta"], stream=stream)
    return C


def test_concurrent_calls_from_host_threads():
    prepared = [_prepare(c, 500 + i) for i, c in enumerate(CASES)]
    streams = [torch.cuda.Stream() for _ in CASES]
    workspaces = []
    for c, (Ad, Bd, C0) in zip(CASES, prepared):
        ws = None
        if c["splitk"]:
            plan = mp.splitk_plan_for(Ad, Bd, C0)
            assert plan["splits"] > 1
            ws = torch.empty(plan["workspace_bytes"] // 4, dtype=torch.float32, device=device())
        workspaces.append(ws)
    torch.cuda.synchronize()
    # each call alone
    alone = []
    for c, (Ad, Bd, C0), s, ws in zip(CASES, prepared, streams, workspaces):
        out = _call(c, Ad, Bd, C0, s, ws)
        s.synchronize()
        alone.append(out.cpu().numpy())
    # all at once, repeatedly
    errors = []
    barrier = threading.Barrier(len(CASES))

    def worker(i):
        try:
            c, (Ad, Bd, C0), s, ws = CASES[i], prepared[i], streams[i], workspaces[i]
            barrier.wait()
            for rep in range(20):
                out = _call(c, Ad, Bd, C0, s, ws)
                s.synchronize()
                if not np.array_equal(out.cpu().numpy(), alone[i]):
                    errors.append(f"case {i} repetition {rep}: differs from the call made alone")
                    return
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(f"case {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
