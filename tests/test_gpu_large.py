"""GPU parity at sizes whose element offsets pass 2^31 (the dimensions and
leading dimensions are 64-bit at the boundary; "any M, N, K" of "Capstone 4:
a tensor-core GEMM", section "Capability").

* C with more than 2^31 elements (about 8.7 GB of FP32), ragged in M and N
  and with a K tail: the tile origins are 64-bit, each wave's stores are
  32-bit offsets from its own tile.  Sampled entries (random, the last rows
  and columns, the corners, every row past the 2^31-element offset) against
  the oracle, every element finite, and the columns between N and ldc
  untouched.
* Leading dimensions so large that one LDS stage of A or of B spans more
  than 32-bit buffer offsets: the factory falls back to the 64-bit direct
  kernel, which must give the oracle's product; the gaps between the rows
  hold NaN, so a read outside the rows shows up.

The large buffers are made on the device (nothing of their size goes
through the host) and freed after each test.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import assert_close, device

pytestmark = pytest.mark.gpu


def test_output_past_2_31_elements():
    M, N, K = 65573, 33005, 21
    ldc = N + 3
    assert M * N > 2 ** 31 and (M - 1) * ldc > 2 ** 31
    dev = device()
    A, B, _ = make_inputs(M, N, K, "uniform", seed=2031)
    Ad, Bd = A.to(dev), B.to(dev)
    flat = torch.full((M * ldc,), float("nan"), dtype=torch.float32, device=dev)
    C = flat.view(M, ldc)[:, :N]
    cfg = mp.query_for(Ad, Bd, C, 1.0, 0.0)
    print(f"[large C] config {cfg['id']} ({cfg['bm']}x{cfg['bn']}), grid {cfg['grid']}", flush=True)
    rng = np.random.default_rng(2031)
    first_far_row = -(-(2 ** 31) // ldc)
    rows = np.concatenate([rng.integers(0, M, 3000), np.arange(first_far_row, M, 7), [M - 1] * 40,
                           [0, 0, M - 1, M - 1], rng.integers(first_far_row, M, 500)])
    cols = np.concatenate([rng.integers(0, N, 3000), rng.integers(0, N, len(range(first_far_row, M, 7))),
                           np.arange(N - 40, N), [0, N - 1, 0, N - 1], [N - 1] * 500])
    ri = torch.as_tensor(rows, device=dev)
    ci = torch.as_tensor(cols, device=dev)
    ref, absdot = oracle.gemm_entries(bits(A), bits(B), None, 1.5, 0.0, rows, cols)

    # beta = 0: C (NaN-poisoned) is not read
    mp.gemm(Ad, Bd, C, 1.5, 0.0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(C).all()), "non-finite output"
    assert bool(torch.isnan(flat.view(M, ldc)[:, N:]).all()), "wrote between N and ldc"
    got = C[ri, ci].cpu().numpy()
    assert_close("large C beta=0", got, ref, absdot, rows, cols)

    # beta = 0.5 on a constant C: the reference is alpha*AB + 0.5*0.25
    C.fill_(0.25)
    mp.gemm(Ad, Bd, C, 1.5, 0.5)
    torch.cuda.synchronize()
    got = C[ri, ci].cpu().numpy()
    assert_close("large C beta=.5", got, ref + 0.125, absdot, rows, cols)
    del flat, C
    torch.cuda.empty_cache()


def _strided_on_device(X, ld, fill):
    """X (rows, cols) copied into a device buffer with leading dimension ld;
    the rest of the buffer holds `fill`."""
    rows, cols = X.shape
    buf = torch.full(((rows - 1) * ld + cols,), fill, dtype=X.dtype, device=device())
    view = torch.as_strided(buf, (rows, cols), (ld, 1))
    view.copy_(X.to(device()))
    return buf, view


@pytest.mark.parametrize("which", ["A", "B"])
def test_stage_span_past_32_bit_offsets_takes_the_direct_kernel(which):
    M, N, K = 70, 50, 40
    A, B, C = make_inputs(M, N, K, "uniform", seed=3131, c_init="uniform")
    big = (1 << 24) + 5            # 64 rows of this stride already span 2^31 bytes
    nan = float("nan")
    if which == "A":
        bufA, Ad = _strided_on_device(A, big, nan)
        Bd = B.to(device())
    else:
        Ad = A.to(device())
        bufB, Bd = _strided_on_device(B, big, nan)
    Cd = C.to(device())
    cfg = mp.query_for(Ad, Bd, Cd, 1.5, 0.5)
    assert cfg["kind_name"] == "direct", cfg
    mp.gemm(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5)
    assert_close(f"huge ld{which.lower()}", Cd.cpu().numpy(), ref, absdot)
    torch.cuda.empty_cache()
