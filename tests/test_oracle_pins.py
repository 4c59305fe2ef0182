"""Pins for the CPU oracle (no GPU).

The oracle is trusted only after it is checked against things other than
itself: a library decoder over every FP16 code, exact rational arithmetic on
tiny shapes, closed forms, values the source pages print, a library FP64
matmul, exact integer products, and symmetry/linearity identities.  The last
tests plant plausible mistakes (on the CPU, in copies of the oracle's output)
and confirm that a pin catches each one.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from dense_mixed_precision_amd.workloads import WORKLOADS, bits, make_inputs, workload_inputs
from tests.exact import exact_gemm, fp64_sum_bound

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))

ALL_CODES = np.arange(65536, dtype=np.uint16)


# ----------------------------------------------------------------------------
# FP16 decoder
# ----------------------------------------------------------------------------

def test_decoder_exhaustive_matches_numpy():
    """All 65,536 bit patterns against numpy's float16 -> float64 conversion."""
    mine = oracle.f16_to_f64(ALL_CODES)
    lib = ALL_CODES.view(np.float16).astype(np.float64)
    nan_mine = np.isnan(mine)
    assert np.array_equal(nan_mine, np.isnan(lib))
    assert nan_mine.sum() == 2 * 1023  # exponent 31 with non-zero fraction, both signs
    fin = ~nan_mine
    assert np.array_equal(mine[fin], lib[fin])
    assert np.array_equal(np.signbit(mine[fin]), np.signbit(lib[fin]))  # -0.0 stays -0.0


def test_decoder_page_values():
    """Largest finite value and the integer grid the pages state."""
    vals = oracle.f16_to_f64(ALL_CODES)
    finite = vals[np.isfinite(vals)]
    assert finite.max() == GOLDEN["fp16_max_finite"]["value"]
    assert oracle.f16_to_f64(np.array([0x7BFF], dtype=np.uint16))[0] == 65504.0
    grid = GOLDEN["fp16_integer_grid"]
    s = set(finite.tolist())
    a, b, c = grid["every_integer_up_to"], grid["every_second_up_to"], grid["every_fourth_up_to"]
    assert all(float(n) in s for n in range(0, a + 1))
    assert all((float(n) in s) == (n % 2 == 0) for n in range(a, b + 1))
    assert all((float(n) in s) == (n % 4 == 0) for n in range(b, c + 1))
    # smallest subnormal and smallest normal
    assert oracle.f16_to_f64(np.array([0x0001], dtype=np.uint16))[0] == 2.0 ** -24
    assert oracle.f16_to_f64(np.array([0x0400], dtype=np.uint16))[0] == 2.0 ** -14


# ----------------------------------------------------------------------------
# Exact brute force on tiny shapes
# ----------------------------------------------------------------------------

def _special_mix(M, K, seed):
    """FP16 bits mixing uniform values with subnormals, tiny normals, signed
    zeros and large magnitudes, so every decoder branch feeds the product."""
    rng = np.random.default_rng(seed)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0xBC00,
                         0x7BFF, 0xFBFF, 0x5800, 0x1400], dtype=np.uint16)
    base = bits(make_inputs(M, K, 1, "uniform", seed)[0])
    mask = rng.random((M, K)) < 0.3
    pick = specials[rng.integers(0, specials.size, (M, K))]
    return np.where(mask, pick, base).astype(np.uint16)


TINY = [(1, 1, 1), (1, 1, 17), (3, 5, 7), (16, 16, 16), (17, 15, 33), (33, 31, 65)]


@pytest.mark.parametrize("M,N,K", TINY)
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5), (-0.75, 2.0)])
def test_brute_force_exact(M, N, K, alpha, beta):
    A, B, C = make_inputs(M, N, K, "uniform", seed=7 * M + N + K, c_init="uniform")
    A_bits, B_bits, C_np = bits(A), bits(B), C.numpy()
    ref, absdot = oracle.gemm(A_bits, B_bits, C_np, alpha, beta)
    eref, eabs, _ = exact_gemm(A_bits, B_bits, C_np, alpha, beta)
    assert np.array_equal(absdot, eabs) or np.allclose(absdot, eabs, rtol=K * 2.0 ** -52, atol=0)
    bound = fp64_sum_bound(K, alpha, beta, eabs, C_np)
    assert np.all(np.abs(ref - eref) <= bound)


@pytest.mark.parametrize("M,N,K", [(16, 16, 16), (17, 15, 33), (9, 11, 40)])
def test_brute_force_special_values(M, N, K):
    A_bits = _special_mix(M, K, seed=M * 100 + K)
    B_bits = _special_mix(K, N, seed=N * 100 + K + 1)
    ref, absdot = oracle.gemm(A_bits, B_bits)
    eref, eabs, _ = exact_gemm(A_bits, B_bits)
    bound = fp64_sum_bound(K, 1.0, 0.0, eabs)
    assert np.all(np.abs(ref - eref) <= bound)


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

def test_all_ones_gives_K():
    M, N, K = 5, 7, 617
    A, B, C = make_inputs(M, N, K, "ones", seed=1, c_init="uniform")
    ref, absdot = oracle.gemm(bits(A), bits(B))
    assert np.all(ref == K) and np.all(absdot == K)
    ref2, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5)
    assert np.array_equal(ref2, 1.5 * K + 0.5 * C.numpy().astype(np.float64))


def test_identity_gives_copy():
    K, N = 64, 37
    A = np.eye(K, dtype=np.float16).view(np.uint16)
    _, B, _ = make_inputs(K, N, K, "uniform", seed=3)
    ref, _ = oracle.gemm(A, bits(B))
    assert np.array_equal(ref, B.numpy().astype(np.float64))


def test_zero_A_and_zero_alpha_give_beta_C():
    M, N, K = 6, 9, 31
    A, B, C = make_inputs(M, N, K, "zeros", seed=2, c_init="uniform", dist_b="uniform")
    c64 = C.numpy().astype(np.float64)
    ref, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.0, 0.5)
    assert np.array_equal(ref, 0.5 * c64)
    A2, _, _ = make_inputs(M, N, K, "uniform", seed=4)
    ref2, _ = oracle.gemm(bits(A2), bits(B), C.numpy(), 0.0, 0.5)
    assert np.array_equal(ref2, 0.5 * c64)


def test_alpha_zero_does_not_read_A_or_B():
    """alpha == 0: the product term is not formed and A and B are not read
    (the counterpart of beta == 0 not reading C), so NaN and Inf in A and B
    do not reach the result: C <- beta*C exactly, sum|ab| reported as 0."""
    M, N, K = 5, 6, 13
    A, B, C = make_inputs(M, N, K, "uniform", seed=8, c_init="uniform")
    A, B = A.clone(), B.clone()
    A[1, 3] = float("nan")
    A[2, 0] = float("inf")
    B[4, 5] = float("-inf")
    B[0, 2] = float("nan")
    c64 = C.numpy().astype(np.float64)
    ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 0.0, 0.5)
    assert np.array_equal(ref, 0.5 * c64) and np.all(absdot == 0)
    poison = np.full((M, N), np.nan, dtype=np.float32)
    ref, _ = oracle.gemm(bits(A), bits(B), poison, 0.0, 0.0)
    assert np.all(ref == 0)
    bias = np.linspace(-1, 1, N, dtype=np.float32)
    ref, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 0.0, -2.0, bias=bias)
    assert np.array_equal(ref, -2.0 * c64 + bias.astype(np.float64)[None, :])
    # with alpha != 0 the same inputs do reach the result
    ref, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.0, 0.5)
    assert np.isnan(ref[1]).all() and np.isnan(ref[:, 2]).all()


def test_k_zero_ignores_alpha():
    """K == 0: no product term, whatever alpha is (Inf or NaN included)."""
    A, B, C = make_inputs(4, 3, 0, "uniform", seed=9, c_init="uniform")
    for alpha in (float("inf"), float("nan"), -3.0):
        ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), alpha, 0.25)
        assert np.array_equal(ref, 0.25 * C.numpy().astype(np.float64)) and np.all(absdot == 0)


def test_beta_zero_does_not_read_C():
    """NaN-poisoned C with beta == 0 must not leak into the result."""
    M, N, K = 8, 8, 8
    A, B, _ = make_inputs(M, N, K, "uniform", seed=5)
    poison = np.full((M, N), np.nan, dtype=np.float32)
    ref, _ = oracle.gemm(bits(A), bits(B), poison, 1.0, 0.0)
    assert np.all(np.isfinite(ref))
    clean, _ = oracle.gemm(bits(A), bits(B))
    assert np.array_equal(ref, clean)


def test_empty_dimensions():
    A, B, C = make_inputs(4, 3, 0, "uniform", seed=6, c_init="uniform")
    ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), 2.0, 0.5)
    assert np.array_equal(ref, 0.5 * C.numpy().astype(np.float64)) and np.all(absdot == 0)
    A, B, _ = make_inputs(0, 3, 5, "uniform", seed=6)
    ref, _ = oracle.gemm(bits(A), bits(B))
    assert ref.shape == (0, 3)


# ----------------------------------------------------------------------------
# Values printed on the pages
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("K", [256, 2048])
def test_largest_small_integer_dot(K):
    g = GOLDEN["small_integer_fill"]
    amax, bmax = g["A_range"][1], g["B_range"][1]
    A = np.full((2, K), amax, dtype=np.float16).view(np.uint16)
    B = np.full((K, 3), bmax, dtype=np.float16).view(np.uint16)
    ref, _ = oracle.gemm(A, B)
    assert amax * bmax == g["largest_product"]
    assert np.all(ref == g["largest_dot"][str(K)])
    A[1] = np.float16(g["A_range"][0]).view(np.uint16)
    ref, _ = oracle.gemm(A, B)
    assert np.all(ref[1] == -g["largest_dot"][str(K)])


def test_k_tail_617_splits_as_608_plus_9():
    g = GOLDEN["k_tail_617"]
    K, head = g["K"], g["full_steps_reach"]
    assert head == (K // g["step"]) * g["step"] and K - head == g["valid_in_last_step"]
    assert g["step"] - g["valid_in_last_step"] == g["past_edge_in_last_step"]
    A, B, _ = make_inputs(23, 19, K, "uniform", seed=617)
    Ab, Bb = bits(A), bits(B)
    full, absdot = oracle.gemm(Ab, Bb)
    p1, a1 = oracle.gemm(np.ascontiguousarray(Ab[:, :head]), np.ascontiguousarray(Bb[:head]))
    p2, a2 = oracle.gemm(np.ascontiguousarray(Ab[:, head:]), np.ascontiguousarray(Bb[head:]))
    assert np.all(np.abs(full - (p1 + p2)) <= fp64_sum_bound(K, 1.0, 0.0, absdot) * 2)
    assert np.allclose(absdot, a1 + a2, rtol=1e-13, atol=0)


# ----------------------------------------------------------------------------
# Library cross-checks and identities
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["square256", "ragged1000x800x617"])
def test_against_numpy_float64_matmul(name):
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    C_np = None if C is None else C.numpy()
    ref, absdot = oracle.gemm(bits(A), bits(B), C_np, w.alpha, w.beta)
    lib = w.alpha * (A.numpy().astype(np.float64) @ B.numpy().astype(np.float64))
    if C is not None and w.beta != 0:
        lib = lib + w.beta * C_np.astype(np.float64)
    bound = 2 * fp64_sum_bound(w.K, w.alpha, w.beta, absdot, C_np)
    assert np.all(np.abs(ref - lib) <= bound)


def test_exact_integers_match_integer_matmul():
    """The pages' exact small-integer fill on a ragged shape: every partial
    sum is an integer below 2^24, so the oracle must equal int64 matmul."""
    M, N, K = 123, 77, 617
    A, B, _ = make_inputs(M, N, K, "smallint", seed=11)
    ref, _ = oracle.gemm(bits(A), bits(B))
    ints = A.numpy().astype(np.int64) @ B.numpy().astype(np.int64)
    assert np.array_equal(ref, ints.astype(np.float64))


def test_transpose_identity_is_bitwise():
    """(B^T A^T)^T = A B with the same products in the same order."""
    A, B, _ = make_inputs(13, 29, 47, "uniform", seed=12)
    Ab, Bb = bits(A), bits(B)
    r1, s1 = oracle.gemm(Ab, Bb)
    r2, s2 = oracle.gemm(np.ascontiguousarray(Bb.T), np.ascontiguousarray(Ab.T))
    assert np.array_equal(r1, r2.T) and np.array_equal(s1, s2.T)


def test_power_of_two_scaling_is_exact():
    A, B, _ = make_inputs(21, 18, 99, "uniform", seed=13)
    r1, _ = oracle.gemm(bits(A), bits(B))
    r2, _ = oracle.gemm(bits(A * 2), bits(B))
    assert np.array_equal(r2, 2 * r1)


def test_strided_leading_dimensions():
    """Views with lda > K, ldb > N and ldc > N give the packed answer."""
    A, B, C = make_inputs(20, 24, 30, "uniform", seed=14, c_init="uniform")
    Ab, Bb, Cn = bits(A), bits(B), C.numpy()
    big_a = np.zeros((20, 37), dtype=np.uint16); big_a[:, :30] = Ab
    big_b = np.zeros((30, 29), dtype=np.uint16); big_b[:, :24] = Bb
    big_c = np.full((20, 31), np.nan, dtype=np.float32); big_c[:, :24] = Cn
    r1, _ = oracle.gemm(Ab, Bb, Cn, 1.25, -0.5)
    r2, _ = oracle.gemm(big_a[:, :30], big_b[:, :24], big_c[:, :24], 1.25, -0.5)
    assert np.array_equal(r1, r2)


def test_entries_match_full_product():
    w = WORKLOADS["ragged1000x800x617"]
    A, B, C = make_inputs(200, 160, 617, "uniform", seed=15, c_init="uniform")
    full, fabs_ = oracle.gemm(bits(A), bits(B), C.numpy(), w.alpha, w.beta)
    rows = np.array([0, 199, 0, 199, 57, 123])
    cols = np.array([0, 159, 159, 0, 81, 2])
    ent, eabs = oracle.gemm_entries(bits(A), bits(B), C.numpy(), w.alpha, w.beta, rows, cols)
    assert np.array_equal(ent, full[rows, cols]) and np.array_equal(eabs, fabs_[rows, cols])


def test_argument_errors():
    A, B, _ = make_inputs(4, 4, 4, "uniform", seed=16)
    with pytest.raises(ValueError):
        oracle.gemm(bits(A), bits(B)[:3])
    with pytest.raises(ValueError):
        oracle.gemm_entries(bits(A), bits(B), None, 1.0, 0.0, [4], [0])
    with pytest.raises(ValueError):
        oracle.gemm(bits(A), bits(B), None, 1.0, 0.5)


# ----------------------------------------------------------------------------
# Column-major operands ("Capstone 4: a tensor-core GEMM", Independent gate:
# A row-major, B column-major; the other combinations follow)
# ----------------------------------------------------------------------------

LAYOUTS = [(0, 1), (1, 0), (1, 1)]


def _stored(X, col_major, pad=0):
    """Logical FP16 bits -> stored array: X itself (row-major) or X^T
    (column-major), optionally inside a wider row so ld exceeds the extent."""
    S = np.ascontiguousarray(X.T) if col_major else X
    if pad:
        big = np.full((S.shape[0], S.shape[1] + pad), 0x7E00, dtype=np.uint16)  # NaN filler
        big[:, :S.shape[1]] = S
        return big[:, :S.shape[1]]
    return S


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 17), (3, 5, 7), (17, 15, 33), (33, 31, 65)])
def test_layout_exact_brute_force(la, lb, M, N, K):
    A, B, C = make_inputs(M, N, K, "uniform", seed=5 * M + 3 * N + K + la + 2 * lb, c_init="uniform")
    Ab, Bb, Cn = bits(A), bits(B), C.numpy()
    ref, absdot = oracle.gemm(_stored(Ab, la), _stored(Bb, lb), Cn, 1.5, 0.5, layout_a=la, layout_b=lb)
    eref, eabs, _ = exact_gemm(Ab, Bb, Cn, 1.5, 0.5)
    assert np.all(np.abs(ref - eref) <= fp64_sum_bound(K, 1.5, 0.5, eabs, Cn))
    assert np.allclose(absdot, eabs, rtol=K * 2.0 ** -52, atol=0)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_layout_matches_row_major_bitwise(la, lb):
    """Same products, same ascending-k order: the stored order must not
    change a single bit, also with leading dimensions beyond the extents
    (the padding holds NaN, so reading it would show)."""
    M, N, K = 37, 29, 83
    A, B, C = make_inputs(M, N, K, "uniform", seed=31 + la + 2 * lb, c_init="uniform")
    Ab, Bb, Cn = bits(A), bits(B), C.numpy()
    r0, s0 = oracle.gemm(Ab, Bb, Cn, -0.75, 2.0)
    r1, s1 = oracle.gemm(_stored(Ab, la, pad=5), _stored(Bb, lb, pad=3), Cn, -0.75, 2.0,
                         layout_a=la, layout_b=lb)
    assert np.array_equal(r0, r1) and np.array_equal(s0, s1)
    rows, cols = np.array([0, M - 1, 5, M - 1]), np.array([0, N - 1, 7, 0])
    e1, _ = oracle.gemm_entries(_stored(Ab, la, pad=5), _stored(Bb, lb, pad=3), Cn, -0.75, 2.0,
                                rows, cols, layout_a=la, layout_b=lb)
    assert np.array_equal(e1, r0[rows, cols])


def test_layout_argument_errors():
    A, B, _ = make_inputs(6, 4, 5, "uniform", seed=17)
    Ab, Bb = bits(A), bits(B)
    with pytest.raises(ValueError):       # stored shapes that do not chain
        oracle.gemm(Ab, Bb, layout_a=1)
    with pytest.raises(ValueError):
        oracle.gemm(Ab, Bb, layout_a=2)
    # column-major A needs lda >= M (checked in the C entry point itself)
    rc = oracle._load().oracle_gemm_layout(1, 0, 6, 4, 5, Ab.ctypes.data, 5, Bb.ctypes.data, 4,
                                           None, 4, 1.0, 0.0, np.empty(24).ctypes.data, None)
    assert rc == -2  # lda = 5 < M = 6 for a column-major A


def test_layout_ignored_is_caught():
    """A plausible slip, reading a column-major operand as if row-major (on a
    square operand, so the shapes still chain), fails the exact pin."""
    M = K = 9
    A, B, _ = make_inputs(M, 7, K, "uniform", seed=18)
    Ab, Bb = bits(A), bits(B)
    wrong, _ = oracle.gemm(_stored(Ab, 1), Bb)        # layout flag dropped
    eref, eabs, _ = exact_gemm(Ab, Bb)
    assert not np.all(np.abs(wrong - eref) <= fp64_sum_bound(K, 1.0, 0.0, eabs))


# ----------------------------------------------------------------------------
# BF16 inputs ("Tensor cores with WMMA", section "A warp owns a tile, and no
# thread owns an element": bf16 is the other 16-bit tensor-core input type)
# ----------------------------------------------------------------------------

def test_bf16_decoder_exhaustive_matches_torch():
    """All 65,536 bit patterns against torch's bfloat16 -> float64 conversion."""
    import torch
    ref = torch.from_numpy(ALL_CODES.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_f64(ALL_CODES)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan]) and np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_decoder_format_values():
    """Values fixed by the format itself (bias 127, 7 fraction bits)."""
    v = oracle.bf16_to_f64(np.array([0x3F80, 0xBF80, 0x4000, 0x3F00, 0x0080, 0x0001, 0x7F7F, 0x8000],
                                    dtype=np.uint16))
    assert v.tolist() == [1.0, -1.0, 2.0, 0.5, 2.0 ** -126, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0]


def _bf16_bits(X):
    import torch
    return X.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16_special_mix(M, K, seed):
    """BF16 bits mixing uniform values with subnormals and far-apart
    exponents, so every decoder branch and a wide exponent range feed the sum."""
    import torch
    rng = np.random.default_rng(seed)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80,
                         0x7F7F, 0xFF7F, 0x5000, 0x2000], dtype=np.uint16)
    base = _bf16_bits(torch.rand(M, K, generator=torch.Generator().manual_seed(seed)) * 2 - 1)
    mask = rng.random((M, K)) < 0.3
    pick = specials[rng.integers(0, specials.size, (M, K))]
    return np.where(mask, pick, base).astype(np.uint16)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 15, 33), (33, 31, 65)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5)])
def test_bf16_brute_force_exact(M, N, K, alpha, beta):
    A, B, C = make_inputs(M, N, K, "uniform", seed=3 * M + N + K, c_init="uniform", dtype=torch_bf16())
    Ab, Bb, Cn = bits(A), bits(B), C.numpy()
    ref, absdot = oracle.gemm(Ab, Bb, Cn, alpha, beta, in_type="bf16")
    eref, eabs, _ = exact_gemm(Ab, Bb, Cn, alpha, beta, in_type="bf16")
    assert np.all(np.abs(ref - eref) <= fp64_sum_bound(K, alpha, beta, eabs, Cn))
    assert np.allclose(absdot, eabs, rtol=K * 2.0 ** -52, atol=0)


@pytest.mark.parametrize("M,N,K", [(16, 16, 16), (9, 11, 40)])
def test_bf16_brute_force_special_values(M, N, K):
    Ab = _bf16_special_mix(M, K, seed=M * 10 + K)
    Bb = _bf16_special_mix(K, N, seed=N * 10 + K + 1)
    ref, _ = oracle.gemm(Ab, Bb, in_type="bf16")
    eref, eabs, _ = exact_gemm(Ab, Bb, in_type="bf16")
    assert np.all(np.abs(ref - eref) <= fp64_sum_bound(K, 1.0, 0.0, eabs))


def test_bf16_matches_f16_where_both_are_exact():
    """Small integers are exact in both formats: the two decoders must give
    the same values, so the two products agree bit for bit."""
    M, N, K = 41, 37, 300
    A, B, _ = make_inputs(M, N, K, "smallint", seed=19)
    r16, s16 = oracle.gemm(bits(A), bits(B))
    rbf, sbf = oracle.gemm(_bf16_bits(A.float()), _bf16_bits(B.float()), in_type="bf16")
    assert np.array_equal(r16, rbf) and np.array_equal(s16, sbf)
    ints = A.numpy().astype(np.int64) @ B.numpy().astype(np.int64)
    assert np.array_equal(rbf, ints.astype(np.float64))


def test_bf16_all_ones_and_layouts():
    M, N, K = 30, 20, 77
    A, B, _ = make_inputs(M, N, K, "ones", seed=1, dtype=torch_bf16())
    ref, _ = oracle.gemm(bits(A), bits(B), in_type="bf16")
    assert np.all(ref == K)
    A, B, C = make_inputs(M, N, K, "uniform", seed=20, c_init="uniform", dtype=torch_bf16())
    r0, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5, in_type="bf16")
    for la, lb in LAYOUTS:
        r1, _ = oracle.gemm(_stored(bits(A), la), _stored(bits(B), lb), C.numpy(), 1.5, 0.5,
                            layout_a=la, layout_b=lb, in_type="bf16")
        assert np.array_equal(r0, r1)


def test_bf16_read_as_f16_is_caught():
    """Decoding BF16 bits with the FP16 decoder (a plausible slip) fails the
    exact pin."""
    A, B, _ = make_inputs(9, 7, 13, "uniform", seed=21, dtype=torch_bf16())
    wrong, _ = oracle.gemm(bits(A), bits(B))   # in_type left at "f16"
    eref, eabs, _ = exact_gemm(bits(A), bits(B), in_type="bf16")
    assert not np.all(np.abs(wrong - eref) <= fp64_sum_bound(13, 1.0, 0.0, eabs))


# ----------------------------------------------------------------------------
# Per-column bias ("Tensor cores with WMMA", section "The habit this API takes
# away": a position-dependent epilogue, a bias per column)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("in_type", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 5), (3, 5, 7), (17, 15, 33)])
def test_bias_exact_brute_force(in_type, M, N, K):
    import torch
    dt = torch.bfloat16 if in_type == "bf16" else torch.float16
    A, B, C = make_inputs(M, N, K, "uniform", seed=M + N + 7 * K, c_init="uniform", dtype=dt)
    bias = np.random.default_rng(M * N).uniform(-1, 1, N).astype(np.float32)
    Ab, Bb, Cn = bits(A), bits(B), C.numpy()
    ref, _ = oracle.gemm(Ab, Bb, Cn, 1.5, 0.5, in_type=in_type, bias=bias)
    eref, eabs, _ = exact_gemm(Ab, Bb, Cn, 1.5, 0.5, in_type=in_type, bias=bias)
    assert np.all(np.abs(ref - eref) <= fp64_sum_bound(K, 1.5, 0.5, eabs, Cn, bias))


def test_bias_closed_forms_and_layouts():
    M, N, K = 12, 9, 20
    A, B, C = make_inputs(M, N, K, "uniform", seed=23, c_init="uniform")
    bias = np.linspace(-2, 2, N).astype(np.float32)
    # zero bias: bit for bit the product without one
    r0, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5)
    rz, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5, bias=np.zeros(N, np.float32))
    assert np.array_equal(r0, rz)
    # alpha = 0: beta*C + bias, each element one FP64 rounding of two exact terms
    ra, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 0.0, 0.5, bias=bias)
    assert np.array_equal(ra, 0.5 * C.numpy().astype(np.float64) + bias.astype(np.float64)[None, :])
    # storage order does not change a bit
    for la, lb in LAYOUTS:
        rl, _ = oracle.gemm(_stored(bits(A), la), _stored(bits(B), lb), C.numpy(), 1.5, 0.5,
                            layout_a=la, layout_b=lb, bias=bias)
        rb, _ = oracle.gemm(bits(A), bits(B), C.numpy(), 1.5, 0.5, bias=bias)
        assert np.array_equal(rl, rb)
    rows, cols = np.array([0, M - 1, 4]), np.array([N - 1, 0, 3])
    e, _ = oracle.gemm_entries(bits(A), bits(B), C.numpy(), 1.5, 0.5, rows, cols, bias=bias)
    assert np.array_equal(e, rb[rows, cols])
    with pytest.raises(ValueError):
        oracle.gemm(bits(A), bits(B), bias=bias[:-1])


def test_bias_by_row_is_caught():
    """Adding bias[i] (the row) instead of bias[j] (a plausible slip) fails
    the exact pin on a non-square output."""
    M, N, K = 5, 8, 11
    A, B, _ = make_inputs(M, N, K, "uniform", seed=24)
    bias = np.arange(N, dtype=np.float32)
    r, _ = oracle.gemm(bits(A), bits(B))
    wrong = r + bias[:M, None].astype(np.float64)
    eref, eabs, _ = exact_gemm(bits(A), bits(B), bias=bias)
    assert not np.all(np.abs(wrong - eref) <= fp64_sum_bound(K, 1.0, 0.0, eabs, None, bias))


def torch_bf16():
    import torch
    return torch.bfloat16


# ----------------------------------------------------------------------------
# The acceptance rule
# ----------------------------------------------------------------------------

def test_tolerance_rule():
    ref = np.zeros(5)
    absdot = np.array([10.0, 10.0, 10.0, 10.0, 0.0])
    tol0 = 1e-3 * 10.0 + 1e-5
    got = np.array([-tol0, 1.01 * tol0, np.nan, np.inf, 1e-5])
    ok = oracle.tolerance_ok(got, ref, absdot)
    assert ok.tolist() == [True, False, False, False, True]


# ----------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------

def _pins_pass(M, N, K, compute):
    """Run a candidate oracle through the exact brute-force pin and the
    transpose pin; True only if both hold."""
    A, B, C = make_inputs(M, N, K, "uniform", seed=99, c_init="uniform")
    Ab, Bb, Cn = bits(A), bits(B), C.numpy()
    ref, _ = compute(Ab, Bb, Cn, 1.5, 0.5)
    eref, eabs, _ = exact_gemm(Ab, Bb, Cn, 1.5, 0.5)
    exact_ok = np.all(np.abs(ref - eref) <= fp64_sum_bound(K, 1.5, 0.5, eabs, Cn))
    r1, _ = compute(Ab, Bb, None, 1.0, 0.0)
    r2, _ = compute(np.ascontiguousarray(Bb.T), np.ascontiguousarray(Ab.T), None, 1.0, 0.0)
    return bool(exact_ok and np.array_equal(r1, r2.T))


def test_real_oracle_passes_the_mutation_harness():
    assert _pins_pass(7, 5, 17, oracle.gemm)


@pytest.mark.parametrize("mistake", ["drop_last_k", "drop_first_k", "sign", "transposed_A",
                                     "beta_ignored", "alpha_ignored", "swapped_alpha_beta"])
def test_planted_mistakes_are_caught(mistake):
    def compute(Ab, Bb, Cn, alpha, beta):
        if mistake == "drop_last_k":
            return oracle.gemm(np.ascontiguousarray(Ab[:, :-1]), np.ascontiguousarray(Bb[:-1]), Cn, alpha, beta)
        if mistake == "drop_first_k":
            return oracle.gemm(np.ascontiguousarray(Ab[:, 1:]), np.ascontiguousarray(Bb[1:]), Cn, alpha, beta)
        if mistake == "sign":
            r, s = oracle.gemm(Ab, Bb, Cn, alpha, beta)
            return -r, s
        if mistake == "transposed_A":
            # reads A[k][i] instead of A[i][k] on a square block
            n = min(Ab.shape)
            At = np.ascontiguousarray(Ab[:n, :n].T)
            Af = Ab.copy(); Af[:n, :n] = At
            return oracle.gemm(Af, Bb, Cn, alpha, beta)
        if mistake == "beta_ignored":
            return oracle.gemm(Ab, Bb, None, alpha, 0.0)
        if mistake == "alpha_ignored":
            return oracle.gemm(Ab, Bb, Cn, 1.0, beta)
        if mistake == "swapped_alpha_beta":
            return oracle.gemm(Ab, Bb, Cn, beta if Cn is not None else alpha, alpha if Cn is not None else beta)
        raise AssertionError(mistake)
    assert not _pins_pass(7, 7, 17, compute)


def test_adversarial_values_against_exact_arithmetic():
    """The pages' adversarial edge values (+-65504, subnormals, the smallest
    normal, zeros, mixed signs and exponents) on a ragged shape: the oracle
    must equal the exact rational result within FP64 summation rounding."""
    M, N, K = 9, 7, 41
    A, B, C = make_inputs(M, N, K, "adversarial", seed=21, c_init="uniform")
    for alpha, beta in ((1.0, 0.0), (1.5, -0.5)):
        ref, absdot = oracle.gemm(bits(A), bits(B), C.numpy(), alpha, beta)
        exact, exact_abs, _ = exact_gemm(bits(A), bits(B), C.numpy(), alpha, beta)
        bound = fp64_sum_bound(K, alpha, beta, exact_abs, C.numpy())
        assert np.all(np.abs(ref - exact) <= bound)
        assert np.allclose(absdot, exact_abs, rtol=1e-15, atol=0)


def test_nonfinite_inputs_follow_ieee():
    """NaN and +-Inf inputs (the pages are silent; IEEE semantics decide):
    the oracle's NaN / +Inf / -Inf pattern equals a plain Python float
    triple loop (IEEE double arithmetic) on the same values, and the finite
    entries agree to FP64 rounding."""
    M, N, K = 6, 5, 9
    A, B, _ = make_inputs(M, N, K, "uniform", seed=31)
    A, B = A.clone(), B.clone()
    A[1, 2] = float("nan")          # row 1 all NaN
    A[3, 4] = float("inf")          # row 3: +-Inf, or NaN where B[4, j] == 0
    B[4, 1] = 0.0
    B[6, 3] = float("-inf")         # column 3: -+Inf, or NaN with row 3's +Inf
    A[0, 6] = 0.0                   # 0 * -Inf = NaN at (0, 3)
    ref, _ = oracle.gemm(bits(A), bits(B))
    a = A.double().tolist()
    b = B.double().tolist()
    want = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += a[i][k] * b[k][j]
            want[i, j] = s
    assert np.array_equal(np.isnan(ref), np.isnan(want))
    assert np.array_equal(np.isposinf(ref), np.isposinf(want))
    assert np.array_equal(np.isneginf(ref), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.allclose(ref[fin], want[fin], rtol=1e-13, atol=1e-15)
    assert np.isnan(ref[1]).all() and np.isnan(ref[0, 3]) and np.isnan(ref[3, 1])


# ----------------------------------------------------------------------------
# The accumulation diagnostic
# ----------------------------------------------------------------------------

def _running_sum(A_bits, B_bits, acc_dtype):
    """C = A @ B with exact products (FP16 x FP16 fits FP32) added one k at a
    time into a running sum rounded to `acc_dtype` after every addition."""
    a = A_bits.view(np.float16).astype(np.float32)
    b = B_bits.view(np.float16).astype(np.float32)
    acc = np.zeros((a.shape[0], b.shape[1]), dtype=acc_dtype)
    for k in range(a.shape[1]):
        acc = (acc.astype(np.float32) + a[:, k:k + 1] * b[k:k + 1, :]).astype(acc_dtype)
    return acc.astype(np.float64)


def test_accumulation_diagnostic_separates_fp32_from_fp16_sums():
    """The pages found that an FP16 accumulator passes the usual checks; the
    acceptance rule is as blind, but the accumulation diagnostic is not.  An
    FP32 running sum stays within the bound; an FP16 running sum of the same
    products passes the acceptance rule on most entries and exceeds the
    bound by far."""
    for dist, K, min_pass in (("uniform", 2048, 1.0), ("normal4", 8192, 0.99)):
        M, N = 8, 32
        A, B, _ = make_inputs(M, N, K, dist, seed=41)
        Ab, Bb = bits(A), bits(B)
        ref, absdot = oracle.gemm(Ab, Bb)
        fp32 = _running_sum(Ab, Bb, np.float32)
        assert oracle.tolerance_ok(fp32, ref, absdot).all()
        assert oracle.accumulation_ratio(fp32, ref, absdot, K, 1.0) <= 0.01
        fp16 = _running_sum(Ab, Bb, np.float16)
        assert oracle.tolerance_ok(fp16, ref, absdot).mean() >= min_pass
        assert oracle.accumulation_ratio(fp16, ref, absdot, K, 1.0) > 2.0


def test_accumulation_bound_terms():
    """Exact results give 0; the bound grows with K, |alpha| and S; NaN in
    the result counts as unbounded; entries whose reference is not finite
    are skipped."""
    ref = np.array([1.0, -2.0, np.inf])
    absdot = np.array([3.0, 3.0, 3.0])
    assert oracle.accumulation_ratio(ref, ref, absdot, 100, 1.5) == 0.0
    b1 = oracle.accumulation_bound(ref[:2], absdot[:2], 100, 1.0)
    assert np.all(oracle.accumulation_bound(ref[:2], absdot[:2], 200, 1.0) > b1)
    assert np.all(oracle.accumulation_bound(ref[:2], absdot[:2], 100, -2.0) > b1)
    got = ref.copy(); got[0] += b1[0] * 0.5
    assert oracle.accumulation_ratio(got, ref, absdot, 100, 1.0) == pytest.approx(0.5)
    got[1] = np.nan
    assert oracle.accumulation_ratio(got, ref, absdot, 100, 1.0) == np.inf
    assert oracle.accumulation_ratio(np.zeros(2), np.zeros(2), np.zeros(2), 0, 1.0) == 0.0


# ----------------------------------------------------------------------------
# The library-matmul form of the full product (for the 8192^3 comparisons)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 15, 33), (33, 31, 65)])
@pytest.mark.parametrize("in_type", ["f16", "bf16"])
def test_matmul_form_against_exact_rationals(M, N, K, in_type):
    """Every layout pair (rows wider than the extents, NaN in the padding),
    with beta and a bias, against exact rational arithmetic (within the FP64
    sum's own rounding bound)."""
    dtype = torch.bfloat16 if in_type == "bf16" else torch.float16
    A, B, C = make_inputs(M, N, K, "uniform", seed=3 * M + K, c_init="uniform", dtype=dtype)
    Ab, Bb, C_np = bits(A), bits(B), C.numpy()
    bias = np.linspace(-1.0, 1.0, N).astype(np.float32)
    eref, eabs, _ = exact_gemm(Ab, Bb, C_np, -0.75, 1.5, in_type=in_type, bias=bias)
    bound = fp64_sum_bound(K, -0.75, 1.5, eabs, C_np, bias)
    for la in (oracle.ROW_MAJOR, oracle.COL_MAJOR):
        for lb in (oracle.ROW_MAJOR, oracle.COL_MAJOR):
            ref, absdot = oracle.gemm_matmul(_stored(Ab, la, pad=3), _stored(Bb, lb, pad=5), C_np, -0.75, 1.5,
                                             layout_a=la, layout_b=lb, in_type=in_type, bias=bias)
            assert np.all(np.abs(ref - eref) <= bound), (la, lb)
            assert np.allclose(absdot, eabs, rtol=(K + 1) * 2.0 ** -52, atol=0), (la, lb)


@pytest.mark.parametrize("name", ["square256", "ragged1000x800x617"])
def test_matmul_form_against_the_loop(name):
    """The two forms of the full product differ only in the order of the
    FP64 additions: within twice the FP64 sum bound of each other."""
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    C_np = None if C is None else C.numpy()
    ref, absdot = oracle.gemm(bits(A), bits(B), C_np, w.alpha, w.beta)
    ref2, absdot2 = oracle.gemm_matmul(bits(A), bits(B), C_np, w.alpha, w.beta)
    bound = 2 * fp64_sum_bound(w.K, w.alpha, w.beta, absdot, C_np)
    assert np.all(np.abs(ref - ref2) <= bound)
    assert np.allclose(absdot, absdot2, rtol=2 * w.K * 2.0 ** -53, atol=0)


def test_matmul_form_exact_integers():
    """Small integers on a ragged shape: every sum is exact, so the result
    equals int64 matmul bit for bit."""
    A, B, _ = make_inputs(123, 77, 617, "smallint", seed=11)
    ref, absdot = oracle.gemm_matmul(bits(A), bits(B))
    ints = A.numpy().astype(np.int64) @ B.numpy().astype(np.int64)
    assert np.array_equal(ref, ints.astype(np.float64))
    assert np.array_equal(absdot, np.abs(A.numpy().astype(np.int64)) @ np.abs(B.numpy().astype(np.int64)))


def test_matmul_form_special_cases():
    """alpha = 0 and K = 0 read neither A nor B (non-finite operands allowed,
    the result is beta*C plus the bias and the sum of |a*b| is 0); beta = 0
    does not read C; otherwise non-finite operands are refused."""
    M, N, K = 6, 9, 31
    A, B, C = make_inputs(M, N, K, "uniform", seed=5, c_init="uniform")
    Ab, Bb, C_np = bits(A).copy(), bits(B), C.numpy()
    Ab[2, 3] = 0x7E00                          # FP16 NaN
    bias = np.arange(N, dtype=np.float32)
    ref, absdot = oracle.gemm_matmul(Ab, Bb, C_np, 0.0, 0.5, bias=bias)
    assert np.array_equal(ref, 0.5 * C_np.astype(np.float64) + bias.astype(np.float64))
    assert np.all(absdot == 0)
    ref0, _ = oracle.gemm(Ab, Bb, C_np, 0.0, 0.5, bias=bias)
    assert np.array_equal(ref, ref0)
    refk, _ = oracle.gemm_matmul(np.zeros((M, 0), np.uint16), np.zeros((0, N), np.uint16), C_np, 1.0, 2.0)
    assert np.array_equal(refk, 2.0 * C_np.astype(np.float64))
    with pytest.raises(ValueError, match="finite"):
        oracle.gemm_matmul(Ab, Bb, C_np, 1.0, 0.5)
    nan_c = np.full((M, N), np.nan, dtype=np.float32)
    r1, _ = oracle.gemm_matmul(bits(A), Bb, nan_c, 1.0, 0.0)
    assert np.all(np.isfinite(r1))


def test_matmul_form_catches_a_transposed_operand():
    """A square B passed in the wrong storage order gives a different
    product, which the comparison with the loop detects."""
    A, B, _ = make_inputs(16, 16, 16, "uniform", seed=9)
    ref, absdot = oracle.gemm(bits(A), bits(B))
    wrong, _ = oracle.gemm_matmul(bits(A), bits(B), layout_b=oracle.COL_MAJOR)
    assert not np.all(np.abs(ref - wrong) <= 2 * fp64_sum_bound(16, 1.0, 0.0, absdot))


def test_accumulation_bound_epilogue_term():
    """beta*c and the bias enter through FP32 roundings whose operands can be
    far larger than the result: with c and the bias cancelling, an exact
    FP32 epilogue (each operation rounded once) stays within the bound only
    with the E = |beta*c| + |bias| term, which covers it."""
    a, b = np.float16(0.0123), np.float16(0.0047)
    s = float(a) * float(b)                        # exact product, K = 1
    c = np.float32(0.7)
    bias = np.float32(-0.7000001)
    ref = s + float(c) + float(bias)               # FP64: exact here
    t = np.float32(np.float32(s) + np.float32(1.0) * c)   # alpha*s + beta*c in FP32
    got = float(np.float32(t + bias))
    absdot = np.array([abs(s)])
    e = oracle.epilogue_abs(1.0, np.array([[c]]), np.array([bias]))
    assert e.shape == (1, 1) and e[0, 0] == abs(float(c)) + abs(float(bias))
    assert oracle.accumulation_ratio(np.array([got]), np.array([ref]), absdot, 1, 1.0) > 1.0
    assert oracle.accumulation_ratio(np.array([got]), np.array([ref]), absdot, 1, 1.0,
                                     epilogue_abs=e.ravel()) <= 1.0


def test_epilogue_abs_forms():
    """Whole-matrix and sampled-entry forms agree; beta = 0 ignores C; no C
    and no bias give 0."""
    rng = np.random.default_rng(3)
    C = rng.uniform(-2, 2, (5, 7)).astype(np.float32)
    bias = rng.uniform(-1, 1, 7).astype(np.float32)
    whole = oracle.epilogue_abs(-0.25, C, bias)
    assert np.array_equal(whole, np.abs(-0.25 * C.astype(np.float64)) + np.abs(bias.astype(np.float64)))
    rows, cols = np.array([0, 4, 2]), np.array([6, 0, 3])
    assert np.array_equal(oracle.epilogue_abs(-0.25, C, bias, rows, cols), whole[rows, cols])
    assert np.array_equal(oracle.epilogue_abs(0.0, C, bias), np.broadcast_to(np.abs(bias.astype(np.float64)), (1, 7)))
    assert oracle.epilogue_abs(0.5, None, None) == 0.0
