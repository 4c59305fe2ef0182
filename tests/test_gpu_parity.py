"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Acceptance (elementwise): |C_gpu - C_ref| <= 1e-3 * sum_k |a_ik b_kj| + 1e-5,
NaN/Inf fail, and the accumulation diagnostic at most 1.  Small and ragged
products are compared on every element here; the large workloads on every
element or whole tiles in test_gpu_fullsize.py, and here also on sampled
entries (one in every 128x128 block, the last row and column, the corners)
plus Freivalds' whole-output check.
Exact-integer, all-ones and identity inputs must match bit for bit.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import WORKLOADS, bits, make_inputs, workload_inputs
from tests.gpu_util import (Guarded, assert_close, device, freivalds_ok, run, run_layout, tile_samples)

pytestmark = pytest.mark.gpu


def _c_np(C):
    return None if C is None else C.numpy()


def full_check(label, A, B, C0, alpha, beta, **kw):
    got, gC = run(A, B, C0, alpha, beta, **kw)
    ref, absdot = oracle.gemm(bits(A), bits(B), _c_np(C0), alpha, beta)
    assert_close(label, got, ref, absdot, K=A.shape[1], alpha=alpha, beta=beta, C0=C0)
    assert gC.untouched_outside_window(), f"{label}: wrote outside the M x N window"
    return got, ref


# ----------------------------------------------------------------------------
# Matrix-core lane layout
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape,nv", [(32, 16), (16, 4)])
def test_mfma_layout_probe(shape, nv):
    out = torch.full((64 * nv,), -1.0, device=device())
    assert mp.mpgemm_probe_mfma_layout(shape, out.data_ptr(), 0) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(64, nv)
    for lane in range(64):
        for v in range(nv):
            if shape == 32:
                row, col = 8 * (v // 4) + 4 * (lane // 32) + v % 4, lane % 32
            else:
                row, col = 4 * (lane // 16) + v, lane % 16
            assert got[lane, v] == row + shape * col, (lane, v, got[lane, v])


@pytest.mark.parametrize("fmt", [mp.MPGEMM_IN_F16, mp.MPGEMM_IN_BF16])
@pytest.mark.parametrize("shape", [32, 16])
def test_mfma_rate_probe_does_the_work_it_counts(shape, fmt):
    # all operands 1: every accumulator element gains the instruction's K
    # (16 or 32) per round, so each lane's sum is exact and known
    dtype = torch.bfloat16 if fmt == mp.MPGEMM_IN_BF16 else torch.float16
    ops = torch.ones(4096, dtype=dtype, device=device())
    wgs, iters = 3, 10
    out = torch.full((wgs * 512,), -1.0, device=device())
    rc = mp.mpgemm_probe_mfma_rate(fmt, shape, ops.data_ptr(), ops.numel(), iters, wgs, out.data_ptr(),
                                   out.numel(), 0)
    assert rc == mp.MPGEMM_OK
    torch.cuda.synchronize()
    per_lane = (8 * 16 * iters * 16) if shape == 32 else (32 * 4 * iters * 32)
    assert torch.all(out == per_lane)


@pytest.mark.parametrize("mode", [mp.MPGEMM_FILL_REG16, mp.MPGEMM_FILL_REG4, mp.MPGEMM_FILL_LDS16])
def test_fill_probe_reads_every_byte_and_reports_clock_spans(mode):
    """The register forms XOR every 32-bit word a thread loads: with each
    word of the buffer equal to its own index, a thread's XOR is known from
    the blocks it reads, so a skipped or misplaced load changes it.  The
    clock spans are ordered, and the shader clock they imply is plausible."""
    MiB = 1 << 20
    words = 8 * MiB // 4
    buf = torch.arange(words, dtype=torch.int32, device=device())
    wgs, depth, footprint = 16, 4, 1 * MiB
    sink = torch.zeros(wgs * 512, dtype=torch.float32, device=device())
    clocks = torch.zeros(wgs * 4, dtype=torch.int64, device=device())
    rc = mp.mpgemm_probe_fill(mode, depth, buf.data_ptr(), words * 4, footprint, 0, 1, 1, wgs, sink.data_ptr(),
                              sink.numel(), clocks.data_ptr(), clocks.numel(), 0)
    assert rc == mp.MPGEMM_OK
    torch.cuda.synchronize()
    c = clocks.view(wgs, 4).cpu().numpy()
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] > c[:, 2]).all()
    ghz = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), ghz
    if mode == mp.MPGEMM_FILL_LDS16:
        assert torch.all(sink == 0)       # the LDS form writes zeros
        return
    # expected XOR per thread: workgroup b on XCD x = b % 8, member j = b // 8;
    # wave u = 8 j + w takes blocks u, u + 8 m, ... (m members per XCD)
    req = 16 if mode == mp.MPGEMM_FILL_REG16 else 4
    blk = 64 * req
    members = wgs // 8
    nblk = footprint // blk
    got = sink.view(torch.int32).cpu().numpy().reshape(wgs, 512)
    for b in (0, 5, wgs - 1):
        x, j = b % 8, b // 8
        for t in (0, 63, 64, 511):
            w, lane = t // 64, t % 64
            u = j * 8 + w
            acc = 0
            for blk_i in range(u, nblk, 8 * members):
                base = (x * footprint + blk_i * blk + lane * req) // 4
                for k in range(req // 4):
                    acc ^= base + k
            assert got[b, t] == np.int32(np.uint32(acc).view(np.int32)), (b, t)


# ----------------------------------------------------------------------------
# The six workloads
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["square256", "ragged1000x800x617", "skinny4096x16x4096"])
def test_workload_every_element(name):
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    print(f"[{name}] {mp.query_for(A.to(device()), B.to(device()), torch.empty(w.M, w.N, device=device()))}",
          flush=True)
    full_check(name, A, B, C, w.alpha, w.beta)


@pytest.mark.parametrize("name", ["square2048", "tallskinny32768x128x4096"])
def test_workload_sampled_and_freivalds(name):
    w = WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    A, B, C = workload_inputs(w)
    got, gC = run(A, B, C, w.alpha, w.beta)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    rows, cols = tile_samples(w.M, w.N, tile=128, per_tile=1, seed=w.seed)
    ref, absdot = oracle.gemm_entries(bits(A), bits(B), _c_np(C), w.alpha, w.beta, rows, cols)
    assert_close(name, got[rows, cols], ref, absdot, rows, cols, K=w.K, alpha=w.alpha, beta=w.beta, C0=C)
    ok, ratio = freivalds_ok(got, A, B, C, w.alpha, w.beta, seed=w.seed)
    print(f"[{name}] {rows.size} sampled entries ok; Freivalds worst ratio {ratio:.3g}", flush=True)
    assert ok, f"{name}: Freivalds check failed (worst err/bound {ratio:.3g})"
    assert gC.untouched_outside_window()


# ----------------------------------------------------------------------------
# Ragged edges, every kernel config, strides and alignment
# ----------------------------------------------------------------------------

EDGE_SHAPES = [
    (1, 1, 1), (1, 1, 17), (15, 17, 16), (16, 16, 16), (17, 15, 33), (31, 33, 65),
    (33, 31, 63), (64, 64, 64), (65, 63, 129), (127, 129, 255), (129, 127, 257),
    (611, 613, 617), (256, 256, 1), (300, 17, 40), (17, 300, 40), (1, 512, 96), (512, 1, 96),
    (4096, 16, 256), (16, 4096, 256),
]


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_edge_shapes_factory(M, N, K):
    A, B, C = make_inputs(M, N, K, "uniform", seed=M * 7 + N * 3 + K, c_init="uniform")
    full_check(f"{M}x{N}x{K} beta=0", A, B, None, 1.0, 0.0)
    full_check(f"{M}x{N}x{K} beta=.5", A, B, C, 1.5, 0.5)


def _pipe_and_direct_ids():
    ids = []
    for i in range(mp.mpgemm_num_configs()):
        c = mp.mpgemm_config_info(i)
        # row-major entries; the column-major ones have their own tests
        if (c["kind_name"] in ("pipe", "direct") and (c["layout_a"], c["layout_b"]) == (0, 0)
                and c["in_type"] == mp.MPGEMM_IN_F16):
            ids.append(i)
    return ids


@pytest.mark.parametrize("cfg", _pipe_and_direct_ids())
def test_every_config_on_ragged_strided_input(cfg):
    """M, N, K fit no tile; lda/ldb are multiples of 8 (so the 16-byte load
    variants apply) but K % 8 and N % 8 leave partial vectors at the edges;
    ldc > N."""
    M, N, K = 261, 147, 101
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg + 100, c_init="uniform")
    full_check(f"config {cfg}", A, B, C, 1.25, -0.75, config=cfg, lda=112, ldb=160, ldc=151)
    full_check(f"config {cfg} beta=0", A, B, None, 1.0, 0.0, config=cfg, lda=112, ldb=160, ldc=149)


@pytest.mark.parametrize("cfg", _pipe_and_direct_ids())
def test_every_config_multi_tile(cfg):
    """Several tiles of every size in both directions and a K loop longer
    than the LDS ring, with exact small integers: must match bit for bit."""
    M, N, K = 520, 600, 392
    A, B, _ = make_inputs(M, N, K, "smallint", seed=cfg + 200)
    got, gC = run(A, B, None, 1.0, 0.0, config=cfg)
    ref, _ = oracle.gemm(bits(A), bits(B))
    assert np.array_equal(got, ref.astype(np.float32)), f"config {cfg}: not bitwise"


def _vector_ids():
    return [i for i in _pipe_and_direct_ids()
            if mp.mpgemm_config_info(i)["kind_name"] == "pipe"
            and (mp.mpgemm_config_info(i)["vec_a"], mp.mpgemm_config_info(i)["vec_b"]) == (8, 8)]


@pytest.mark.parametrize("cfg", _vector_ids())
def test_every_vector_config_on_unaligned_operands(cfg):
    """The 16-byte copy paths on operands that are only 2-byte aligned:
    offset base pointers and odd leading dimensions, so every row of A and B
    starts at a different alignment."""
    M, N, K = 261, 147, 101
    A, B, C = make_inputs(M, N, K, "uniform", seed=cfg + 300, c_init="uniform")
    full_check(f"config {cfg} unaligned", A, B, C, 1.25, -0.75, config=cfg,
               a_off=1, b_off=3, lda=103, ldb=149, ldc=151)


def test_misaligned_pointers_and_odd_leading_dimensions():
    M, N, K = 333, 250, 617
    A, B, C = make_inputs(M, N, K, "uniform", seed=41, c_init="uniform")
    for a_off, b_off, lda, ldb in [(1, 0, K, N), (0, 1, K, N), (1, 1, K + 3, N + 5), (0, 0, K, N + 1)]:
        full_check(f"a_off={a_off} b_off={b_off} lda={lda} ldb={ldb}", A, B, C, 1.5, 0.5,
                   a_off=a_off, b_off=b_off, lda=lda, ldb=ldb)


# ----------------------------------------------------------------------------
# Exact cases
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1000, 800, 617), (333, 257, 129), (256, 256, 256), (64, 4096, 2048)])
def test_small_integers_bitwise(M, N, K):
    A, B, _ = make_inputs(M, N, K, "smallint", seed=M + N + K)
    got, _ = run(A, B, None, 1.0, 0.0)
    ref, _ = oracle.gemm(bits(A), bits(B))
    assert np.array_equal(got, ref.astype(np.float32))


def test_all_ones_gives_K_and_identity_gives_copy():
    M, N, K = 300, 200, 617
    A, B, _ = make_inputs(M, N, K, "ones", seed=1)
    got, _ = run(A, B, None, 1.0, 0.0)
    assert np.all(got == K)
    Kq = 300
    I = torch.eye(Kq, dtype=torch.float16)
    _, B2, _ = make_inputs(Kq, 211, Kq, "uniform", seed=2)
    got, _ = run(I, B2, None, 1.0, 0.0)
    assert np.array_equal(got, B2.numpy().astype(np.float32))


def test_alpha_zero_and_k_zero_scale_C():
    M, N = 130, 70
    A, B, C = make_inputs(M, N, 33, "uniform", seed=3, c_init="uniform")
    got, _ = run(A, B, C, 0.0, 0.5)
    assert np.array_equal(got, (np.float32(0.5) * C.numpy()))
    A0, B0, _ = make_inputs(M, N, 0, "uniform", seed=3)
    got, _ = run(A0, B0, C, 1.0, -2.0)
    assert np.array_equal(got, (np.float32(-2.0) * C.numpy()))
    got, _ = run(A0, B0, None, 1.0, 0.0)
    assert np.all(got == 0)


def test_alpha_zero_and_k_zero_do_not_read_A_or_B():
    """alpha == 0 (or K == 0, whatever alpha is) means A and B are not read:
    NaN and Inf in them do not reach C, which becomes beta*C (+ bias), as
    the oracle computes it (the reading both take where the pages are
    silent), bit for bit.  Through the plain, the bias and the split-K
    entry points."""
    M, N, K = 130, 70, 33
    A, B, C = make_inputs(M, N, K, "uniform", seed=13, c_init="uniform")
    A, B = A.clone(), B.clone()
    A[3, 5] = float("nan")
    A[100, 0] = float("inf")
    B[7, 69] = float("-inf")
    B[32, 1] = float("nan")
    for beta in (0.5, -2.0):
        ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 0.0, beta)
        assert np.all(absdot == 0)
        got, _ = run(A, B, C, 0.0, beta)
        assert np.array_equal(got, ref.astype(np.float32)), f"beta={beta}: differs from beta*C"
    bias = np.linspace(-1, 1, N).astype(np.float32)
    ref, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 0.0, 0.5, bias=bias)
    got, _ = run_layout(A, B, C, 0.0, 0.5, 0, 0, bias=bias)
    assert np.array_equal(got, ref.astype(np.float32))
    # split-K entry point: a product it would split, with alpha == 0
    Ad, Bd = A.to(device()), B.to(device())
    Cd = C.to(device())
    mp.gemm_splitk(Ad, Bd, Cd, 0.0, 0.5, splits=4)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 0.0, 0.5)
    assert np.array_equal(Cd.cpu().numpy(), ref.astype(np.float32))
    # K == 0 with a non-finite alpha: C <- beta*C; beta == 0 writes zeros over NaN
    A0, B0, _ = make_inputs(M, N, 0, "uniform", seed=14)
    for alpha in (float("inf"), float("nan")):
        ref, _ = oracle.gemm(bits(A0), bits(B0), C.numpy(), alpha, 0.25)
        got, _ = run(A0, B0, C, alpha, 0.25)
        assert np.array_equal(got, ref.astype(np.float32)), alpha
    got, _ = run(A, B, None, 0.0, 0.0, poison=True)
    assert np.all(got == 0)


def test_nan_poisoned_C_is_not_read_when_beta_is_zero():
    M, N, K = 257, 255, 129
    A, B, _ = make_inputs(M, N, K, "uniform", seed=4)
    got, _ = run(A, B, None, 1.0, 0.0, poison=True)
    assert np.all(np.isfinite(got))


def test_deterministic_bitwise_across_runs():
    w = WORKLOADS["ragged1000x800x617"]
    A, B, C = workload_inputs(w)
    g1, _ = run(A, B, C, w.alpha, w.beta)
    g2, _ = run(A, B, C, w.alpha, w.beta)
    assert np.array_equal(g1, g2)
    A, B, _ = make_inputs(2048, 2048, 2048, "uniform", seed=5)
    g1, _ = run(A, B, None, 1.0, 0.0)
    g2, _ = run(A, B, None, 1.0, 0.0)
    assert np.array_equal(g1, g2)


def test_non_default_stream():
    M, N, K = 640, 384, 200
    A, B, C = make_inputs(M, N, K, "uniform", seed=6, c_init="uniform")
    s = torch.cuda.Stream()
    full_check("side stream", A, B, C, 1.0, 1.0, stream=s)


def test_an_earlier_runtime_error_is_not_reported_as_this_calls():
    """A failed HIP call made before (here an allocation far beyond the
    device, refused on the host) leaves the runtime's last error set; the
    library's calls must still report their own outcome, on the scale-only
    path (alpha = 0) as on the product path."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime already in the process
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMalloc.restype = ctypes.c_int
    M, N, K = 70, 50, 40
    A, B, C = make_inputs(M, N, K, "uniform", seed=77, c_init="uniform")
    Ad, Bd, Cd = A.to(device()), B.to(device()), C.to(device())
    for alpha, beta in ((0.0, 0.5), (1.0, 0.5)):
        ptr = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(ptr), 1 << 60) != 0
        rc = mp.mpgemm_f16f32(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, Cd.data_ptr(), N, alpha, beta,
                              torch.cuda.current_stream().cuda_stream)
        assert rc == mp.MPGEMM_OK, (alpha, mp.mpgemm_strerror(rc))
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm(bits(A), bits(B), (np.float32(0.5) * C.numpy()), 1.0, 0.5)
    assert_close("after stale errors", Cd.cpu().numpy(), ref, absdot, K=K, alpha=1.0)
