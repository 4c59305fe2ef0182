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
  than 32-bit buffer offsets: the factory falls back to a tiled entry whose
  stages still fit (16-row tiles), or else to the 64-bit direct kernel;
  either must give the oracle's product; the gaps between the rows hold
  NaN, so a read outside the rows shows up.
* K = 2^31 + 9 through split-K, exact.

The large buffers are made on the device and freed after each test; only
the split-K case copies its two 4.3 GB operands to the host, for the
oracle.
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
    assert_close("large C beta=0", got, ref, absdot, rows, cols, K=K, alpha=1.5)

    # beta = 0.5 on a constant C: the reference is alpha*AB + 0.5*0.25
    C.fill_(0.25)
    mp.gemm(Ad, Bd, C, 1.5, 0.5)
    torch.cuda.synchronize()
    got = C[ri, ci].cpu().numpy()
    assert_close("large C beta=.5", got, ref + 0.125, absdot, rows, cols, K=K, alpha=1.5, beta=0.5,
                 C0=np.broadcast_to(np.float32(0.25), (M, N)))
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


@pytest.mark.parametrize("which,big,kind", [
    ("A", (1 << 24) + 5, "pipe"),    # 64 rows of this stride span 2^31 bytes, 16 rows do not
    ("A", (1 << 26) + 5, "direct"),  # 16 rows of this stride already span 2^31 bytes
    ("B", (1 << 24) + 5, "direct"),  # 64 k rows of this stride span 2^31 bytes
])
def test_stage_span_past_32_bit_offsets_takes_a_kernel_that_fits(which, big, kind):
    """Leading dimensions so large that a tile's stage overflows 32-bit
    buffer offsets: the factory takes a tiled entry whose stages still fit
    (the 16-row tiles), else the 64-bit direct kernel."""
    M, N, K = 70, 50, 40
    A, B, C = make_inputs(M, N, K, "uniform", seed=3131, c_init="uniform")
    nan = float("nan")
    print(f"[huge ld{which.lower()} {big}] {M}x{N}x{K}", flush=True)
    if which == "A":
        bufA, Ad = _strided_on_device(A, big, nan)
        Bd = B.to(device())
    else:
        Ad = A.to(device())
        bufB, Bd = _strided_on_device(B, big, nan)
    Cd = C.to(device())
    cfg = mp.query_for(Ad, Bd, Cd, 1.5, 0.5)
    assert cfg["kind_name"] == kind, cfg
    if kind == "pipe":
        assert (cfg["bm"] * big + cfg["bk"]) * 2 < 0x7FFFFFF0, cfg
    mp.gemm(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5)
    assert_close(f"huge ld{which.lower()}", Cd.cpu().numpy(), ref, absdot, K=K, alpha=1.5)
    torch.cuda.empty_cache()


def test_k_past_2_31_through_split_k():
    """K = 2^31 + 9 for a 1 x 1 output, through split-K (one tile, so the plan
    cuts K into pieces; 64-bit K offsets per piece, a K tail in the last).
    A is the 1 x K row stored column-major (lda = 1; stored row-major its
    leading dimension K would put a stage past 32-bit offsets, which the
    64-bit direct kernel takes unsplit), B is K x 1 row-major.  Values in
    {-1, 0, 1}: every partial sum is an integer far below 2^24 in magnitude
    (a random walk of 2^31 steps stays within a few times 4e4), so the FP32
    result is exact and must equal the oracle's bit for bit."""
    K = 2 ** 31 + 9
    dev = device()
    g = torch.Generator(device=dev)
    g.manual_seed(2311)
    # drawn on the device (seeded), copied to the host for the oracle
    Ad = torch.randint(-1, 2, (K,), generator=g, device=dev, dtype=torch.int8).to(torch.float16)
    Bd = torch.randint(-1, 2, (K,), generator=g, device=dev, dtype=torch.int8).to(torch.float16)
    a = Ad.cpu().numpy()
    b = Bd.cpu().numpy()
    C = torch.full((1,), float("nan"), device=dev)
    args = (mp.MPGEMM_IN_F16, mp.MPGEMM_COL_MAJOR, mp.MPGEMM_ROW_MAJOR, 1, 1, K, Ad.data_ptr(), 1,
            Bd.data_ptr(), 1)
    plan = mp.mpgemm_splitk_plan(*args, 0)
    print(f"[K=2^31+9] split-K plan {plan}", flush=True)
    assert plan["splits"] > 1 and mp.mpgemm_config_info(plan["config_id"])["kind_name"] == "pipe"
    ws = torch.empty(plan["workspace_bytes"] // 4, dtype=torch.float32, device=dev)
    rc = mp.mpgemm_gemm_splitk(*args, C.data_ptr(), 1, 1.0, 0.0, 0, 0, ws.data_ptr(), ws.numel() * 4,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == mp.MPGEMM_OK, mp.mpgemm_strerror(rc)
    torch.cuda.synchronize()
    # The oracle's dot product in 256 blocks of 2^23 values (the diagonal
    # entries of the block-reshaped product, computed in parallel) plus the
    # 9-value remainder: integer partial results, so their FP64 sum is exact.
    R, L = 256, 2 ** 23
    ab, bb = a.view(np.uint16), b.view(np.uint16)
    diag = np.arange(R)
    blocks, _ = oracle.gemm_entries(ab[:R * L].reshape(R, L), bb[:R * L].reshape(R, L), None, 1.0, 0.0,
                                    diag, diag, layout_b=oracle.COL_MAJOR)
    rest, _ = oracle.gemm(ab[R * L:].reshape(1, K - R * L), bb[R * L:].reshape(K - R * L, 1))
    ref = float(np.sum(blocks)) + float(rest[0, 0])
    got = C.cpu().numpy()
    assert got[0] == np.float32(ref), (got[0], ref)
    del Ad, Bd, C, ws
    torch.cuda.empty_cache()
