"""GPU parity of every operand form the benchmark times, at the benchmark's
sizes and in its launch configuration (the factory's choice): the 2048^3 and
8192^3 workloads with B column-major, A and B column-major, BF16 inputs
(row-major and B column-major), and a per-column bias.

Every element is compared with the oracle, within |C - C_ref| <= 1e-3 * S
+ 1e-5 and the accumulation diagnostic: at 2048^3 against the oracle's C
loop, at 8192^3 against its library-matmul form (the loop would take about
half an hour there), plus, against the loop, every element of the first and
last rows and columns.  Both also get Freivalds' check over the whole
output: for a random +-1 vector x,
row i of C@x - (alpha*A@(B@x) + bias*sum(x)) is a signed sum of the row's
element errors, so it is bounded by 1e-3*(|A|@(|B|@|x|))_i + 1e-5*N when
every element is within tolerance.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import WORKLOADS, bits, workload_inputs
from tests.gpu_util import assert_close, run_layout, stored

pytestmark = pytest.mark.gpu

VARIANTS = [(0, 1, "f16", False), (1, 1, "f16", False), (0, 0, "bf16", False), (0, 1, "bf16", False),
            (0, 0, "f16", True)]


def freivalds(got, A, B, alpha, bias, seed):
    rng = np.random.default_rng(seed)
    N = got.shape[1]
    x = rng.choice([-1.0, 1.0], size=N)
    A64 = A.to(torch.float64).numpy()
    B64 = B.to(torch.float64).numpy()
    lhs = got.astype(np.float64) @ x
    rhs = float(np.float32(alpha)) * (A64 @ (B64 @ x))
    if bias is not None:
        rhs = rhs + float(bias.astype(np.float64) @ x)
    S = np.abs(A64) @ (np.abs(B64) @ np.abs(x))
    bound = 1e-3 * S + 1e-5 * N + 1e-9 * (S + np.abs(got).astype(np.float64) @ np.abs(x))
    err = np.abs(lhs - rhs)
    return bool(np.all(err <= bound)), float(np.max(err / bound))


def query(w, la, lb, fmt):
    """The factory's choice for the workload in this operand form (no launch;
    stand-in pointers, which the query only checks for alignment)."""
    fn = mp.mpgemm_bf16f32_layout_query if fmt == "bf16" else mp.mpgemm_f16f32_layout_query
    lda = w.M if la else w.K
    ldb = w.K if lb else w.N
    return fn(la, lb, w.M, w.N, w.K, 1 << 20, lda, 1 << 21, ldb, 1 << 22, w.N, w.alpha, w.beta)


@pytest.mark.parametrize("la,lb,fmt,with_bias", VARIANTS)
@pytest.mark.parametrize("name", ["square2048", "square8192"])
def test_bench_variant_parity(name, la, lb, fmt, with_bias):
    w = WORKLOADS[name]
    dtype = torch.bfloat16 if fmt == "bf16" else torch.float16
    label = f"{name} A{'col' if la else 'row'} B{'col' if lb else 'row'} {fmt}{' bias' if with_bias else ''}"
    print(f"[{label}] generating inputs", flush=True)
    A, B, _ = workload_inputs(w, dtype)
    bias = None
    if with_bias:
        g = torch.Generator().manual_seed(w.seed + 77)
        bias = (torch.rand(w.N, generator=g) * 2 - 1).numpy().astype(np.float32)
    got, gC = run_layout(A, B, None, w.alpha, w.beta, la, lb, bias=bias)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert gC.untouched_outside_window()
    As, Bs = bits(stored(A, la)), bits(stored(B, lb))
    opts = dict(layout_a=la, layout_b=lb, in_type=fmt, bias=bias)
    if name == "square2048":
        print(f"[{label}] oracle over all {w.M * w.N} entries", flush=True)
        ref, absdot = oracle.gemm(As, Bs, None, w.alpha, w.beta, **opts)
        assert_close(label, got, ref, absdot, K=w.K, alpha=w.alpha, bias=bias)
    else:
        cfg = query(w, la, lb, fmt)
        assert (cfg["bm"], cfg["bn"], cfg["grid"]) == (256, 256, 1024)
        print(f"[{label}] oracle (library-matmul form) over all {w.M * w.N} entries", flush=True)
        ref, absdot = oracle.gemm_matmul(As, Bs, None, w.alpha, w.beta, **opts)
        assert_close(label, got, ref, absdot, K=w.K, alpha=w.alpha, bias=bias)
        del ref, absdot
        rows = np.concatenate([np.zeros(w.N), np.full(w.N, w.M - 1), np.arange(w.M),
                               np.arange(w.M)]).astype(np.int64)
        cols = np.concatenate([np.arange(w.N), np.arange(w.N), np.zeros(w.M),
                               np.full(w.M, w.N - 1)]).astype(np.int64)
        ref, absdot = oracle.gemm_entries(As, Bs, None, w.alpha, w.beta, rows, cols, **opts)
        assert_close(f"{label} edge rows/columns", got[rows, cols], ref, absdot, rows, cols, K=w.K,
                     alpha=w.alpha, bias=bias)
    ok, ratio = freivalds(got, A, B, w.alpha, bias, seed=w.seed)
    print(f"[{label}] Freivalds worst ratio {ratio:.3g}", flush=True)
    assert ok, f"{label}: Freivalds check failed (worst err/bound {ratio:.3g})"
