"""CPU oracle for the FP16-input, FP32-accumulate GEMM  C = alpha*A@B + beta*C.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``dense_mixed_precision_amd``) never imports it, and the two share no code:
the arithmetic lives in ``oracle.c`` (plain C, FP64), built by :func:`build`
with gcc into ``liboracle.so`` and called here through ctypes.

What it computes is the plain definition of the product ("Capstone 4: a
tensor-core GEMM", Minimal model and Compare like with like): FP16 inputs
widened exactly to FP64, products exact, the sum carried in FP64 in ascending
k, then ``alpha*s + beta*c`` with C not read when ``beta == 0``, and A and B
not read when ``alpha == 0`` or ``K == 0`` (then the result is ``beta*c``).

The acceptance rule for a GPU result ``c`` against this oracle is
``|c - ref| <= 1e-3 * sum_k|a_ik*b_kj| + 1e-5`` elementwise (see
:func:`tolerance_ok`); the oracle returns that sum alongside the result.
:func:`accumulation_ratio` is a second, diagnostic check: the error against
the worst case of an FP32 running sum, which an FP16 running sum exceeds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

#: gcc flags: no fast-math, no contraction, so the FP64 sum is evaluated
#: exactly as written (ascending k, separate multiply and add).
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared"]

# Relative and absolute terms of the acceptance rule.
TOL_REL = 1e-3
TOL_ABS = 1e-5

_lib = None


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (always recompiles)."""
    global _lib
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f64_array.argtypes = [vp, i64, vp]
    lib.oracle_f16_to_f64_array.restype = None
    lib.oracle_gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                ctypes.c_double, ctypes.c_double, vp, vp]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                        ctypes.c_double, ctypes.c_double,
                                        i64, vp, vp, vp, vp]
    lib.oracle_gemm_entries.restype = ctypes.c_int
    lib.oracle_gemm_layout.argtypes = [ctypes.c_int, ctypes.c_int] + lib.oracle_gemm.argtypes
    lib.oracle_gemm_layout.restype = ctypes.c_int
    lib.oracle_gemm_layout_entries.argtypes = [ctypes.c_int, ctypes.c_int] + lib.oracle_gemm_entries.argtypes
    lib.oracle_gemm_layout_entries.restype = ctypes.c_int
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64_array.argtypes = [vp, i64, vp]
    lib.oracle_bf16_to_f64_array.restype = None
    lib.oracle_gemm_bf16_layout.argtypes = lib.oracle_gemm_layout.argtypes
    lib.oracle_gemm_bf16_layout.restype = ctypes.c_int
    lib.oracle_gemm_bf16_layout_entries.argtypes = lib.oracle_gemm_layout_entries.argtypes
    lib.oracle_gemm_bf16_layout_entries.restype = ctypes.c_int
    lib.oracle_gemm_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, i64,
                                   vp, i64, vp, i64, ctypes.c_double, ctypes.c_double, vp, vp, vp]
    lib.oracle_gemm_ex.restype = ctypes.c_int
    lib.oracle_gemm_ex_entries.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                           vp, i64, vp, i64, vp, i64, ctypes.c_double,
                                           ctypes.c_double, vp, i64, vp, vp, vp, vp]
    lib.oracle_gemm_ex_entries.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all host cores)."""
    return int(_load().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_bits_2d(x, name):
    """Return (array, leading dimension) for a 2-D uint16 row-major view
    (FP16 or BF16 bit patterns)."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float16 or uint16 (16-bit patterns) array")
    if x.size == 0:
        return np.zeros(x.shape, dtype=np.uint16), max(x.shape[1], 1)
    # a dimension of extent 1 has no meaningful stride (numpy may report any)
    if (x.shape[1] > 1 and x.strides[1] != 2) or (x.shape[0] > 1 and (x.strides[0] % 2 or x.strides[0] <= 0)):
        raise ValueError(f"{name} must be row-major with unit inner stride")
    ld = max(x.strides[0] // 2 if x.shape[0] > 1 else 0, max(x.shape[1], 1))
    return x, ld


def _as_c(C, M, N, beta):
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        return None, max(N, 1)
    C = np.asarray(C)
    if C.dtype != np.float32 or C.ndim != 2 or C.shape != (M, N):
        raise TypeError("C must be a float32 array of shape (M, N)")
    if (N > 1 and C.strides[1] != 4) or (M > 1 and (C.strides[0] % 4 or C.strides[0] <= 0)):
        raise ValueError("C must be row-major with unit inner stride")
    return C, max(C.strides[0] // 4 if M > 1 else 0, max(N, 1))


def f16_to_f64(bits) -> np.ndarray:
    """Decode FP16 bit patterns to FP64 with the oracle's own decoder."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_f16_to_f64_array(_ptr(bits), bits.size, _ptr(out))
    return out


#: Storage orders of A and B (C is always row-major).
ROW_MAJOR = 0
COL_MAJOR = 1


def _operands(A, B, layout_a, layout_b):
    """Stored arrays and their leading dimensions -> (A, lda, B, ldb, M, N, K).

    A is stored (M, K) when row-major and (K, M) when column-major; B is
    stored (K, N) when row-major and (N, K) when column-major."""
    if layout_a not in (ROW_MAJOR, COL_MAJOR) or layout_b not in (ROW_MAJOR, COL_MAJOR):
        raise ValueError("layouts must be ROW_MAJOR (0) or COL_MAJOR (1)")
    A, lda = _as_bits_2d(A, "A")
    B, ldb = _as_bits_2d(B, "B")
    M, K = A.shape if layout_a == ROW_MAJOR else A.shape[::-1]
    K2, N = B.shape if layout_b == ROW_MAJOR else B.shape[::-1]
    if K2 != K:
        raise ValueError("inner dimensions differ")
    return A, lda, B, ldb, M, N, K


def bf16_to_f64(bits) -> np.ndarray:
    """Decode BF16 bit patterns to FP64 with the oracle's own decoder."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_bf16_to_f64_array(_ptr(bits), bits.size, _ptr(out))
    return out


#: Input formats of A and B: "f16" (IEEE binary16) or "bf16" (bfloat16).
IN_TYPES = ("f16", "bf16")


def _bf16_flag(in_type):
    if in_type not in IN_TYPES:
        raise ValueError(f"in_type must be one of {IN_TYPES}")
    return 1 if in_type == "bf16" else 0


def _as_bias(bias, N):
    """Per-column bias: None, or N float32 values (contiguous)."""
    if bias is None:
        return None
    bias = np.ascontiguousarray(np.asarray(bias), dtype=np.float32)
    if bias.shape != (N,):
        raise ValueError(f"bias must hold N = {N} values")
    return bias


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")


def gemm(A, B, C=None, alpha: float = 1.0, beta: float = 0.0,
         layout_a: int = ROW_MAJOR, layout_b: int = ROW_MAJOR, in_type: str = "f16", bias=None):
    """Full product.  Returns ``(ref, absdot)``, both float64 (M, N).

    A: 16-bit patterns (FP16, or BF16 with ``in_type="bf16"``) stored (M, K)
    (row-major) or (K, M) (``layout_a=COL_MAJOR``); B: stored (K, N) or (N, K)
    (``layout_b=COL_MAJOR``); C: (M, N) float32 or None; bias: N float32
    values added to every row, or None.  alpha and beta are rounded to
    float32 first, as the GPU entry point receives them.
    """
    flag = _bf16_flag(in_type)
    A, lda, B, ldb, M, N, K = _operands(A, B, layout_a, layout_b)
    bias = _as_bias(bias, N)
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    C, ldc = _as_c(C, M, N, beta)
    ref = np.empty((M, N), dtype=np.float64)
    absdot = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_gemm_ex(flag, layout_a, layout_b, M, N, K, _ptr(A), lda, _ptr(B), ldb,
                                  _ptr(C), ldc, alpha, beta, _ptr(bias), _ptr(ref), _ptr(absdot)))
    return ref, absdot


def gemm_entries(A, B, C, alpha: float, beta: float, rows, cols,
                 layout_a: int = ROW_MAJOR, layout_b: int = ROW_MAJOR, in_type: str = "f16",
                 bias=None):
    """Selected entries (rows[t], cols[t]).  Returns ``(ref, absdot)`` 1-D.
    Operands as for :func:`gemm`."""
    flag = _bf16_flag(in_type)
    A, lda, B, ldb, M, N, K = _operands(A, B, layout_a, layout_b)
    bias = _as_bias(bias, N)
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    C, ldc = _as_c(C, M, N, beta)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and equal length")
    ref = np.empty(rows.shape, dtype=np.float64)
    absdot = np.empty(rows.shape, dtype=np.float64)
    _check(_load().oracle_gemm_ex_entries(flag, layout_a, layout_b, M, N, K, _ptr(A), lda, _ptr(B),
                                          ldb, _ptr(C), ldc, alpha, beta, _ptr(bias), rows.size,
                                          _ptr(rows), _ptr(cols), _ptr(ref), _ptr(absdot)))
    return ref, absdot


def gemm_matmul(A, B, C=None, alpha: float = 1.0, beta: float = 0.0,
                layout_a: int = ROW_MAJOR, layout_b: int = ROW_MAJOR, in_type: str = "f16", bias=None):
    """The same full product as :func:`gemm`, with the K-sums taken by a
    library FP64 matrix product (numpy's ``@``) instead of the C loop, for
    sizes the loop cannot finish in a test's time (8192^3: about half an hour
    on 8 cores for the loop, seconds for the library product).  Returns ``(ref,
    absdot)`` like :func:`gemm`, with the same conventions (operands,
    layouts, bias, alpha and beta rounded to float32, C not read when
    ``beta == 0``, A and B not read when ``alpha == 0`` or ``K == 0``).

    It is still the plain definition ("Capstone 4: a tensor-core GEMM",
    Compare like with like: every element against the double-precision
    result): the inputs are widened exactly by the oracle's own decoders,
    every product of two widened inputs is exact in FP64, and only the order
    in which the library adds them differs from the loop's ascending k, so
    each sum is within K * 2^-53 * S of the exact one on both paths
    (S = sum_k |a_ik b_kj|) and the two agree to 2 * K * 2^-53 * S, eight
    orders of magnitude inside the acceptance tolerance at K = 8192.  The
    library product does not promise the loop's handling of Inf and NaN, so
    operands that are read must be finite (``ValueError`` otherwise; use
    :func:`gemm` for non-finite inputs)."""
    _bf16_flag(in_type)
    A, _, B, _, M, N, K = _operands(A, B, layout_a, layout_b)
    bias = _as_bias(bias, N)
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    C, _ = _as_c(C, M, N, beta)
    ref = np.zeros((M, N), dtype=np.float64)
    absdot = np.zeros((M, N), dtype=np.float64)
    if alpha != 0.0 and K > 0 and M > 0 and N > 0:
        decode = bf16_to_f64 if in_type == "bf16" else f16_to_f64
        a = decode(A)
        b = decode(B)
        if not (np.all(np.isfinite(a)) and np.all(np.isfinite(b))):
            raise ValueError("gemm_matmul needs finite A and B; use gemm for Inf or NaN inputs")
        if layout_a == COL_MAJOR:
            a = a.T
        if layout_b == COL_MAJOR:
            b = b.T
        ref = alpha * (a @ b)
        absdot = np.abs(a) @ np.abs(b)
    if beta != 0.0:
        ref = ref + beta * C.astype(np.float64)
    if bias is not None:
        ref = ref + bias.astype(np.float64)[None, :]
    return ref, absdot


def tolerance_ok(got, ref, absdot):
    """Elementwise acceptance: ``|got - ref| <= 1e-3*absdot + 1e-5``.

    The comparison is ``err <= tol``, which is False for NaN, so NaN or Inf in
    ``got`` fails.  Returns a boolean array of the broadcast shape.
    """
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    tol = TOL_REL * absdot + TOL_ABS
    return err <= tol


#: FP32 unit roundoff (round to nearest) and smallest normal.
U_FP32 = 2.0 ** -24
TINY_FP32 = 2.0 ** -126


def accumulation_bound(ref, absdot, K: int, alpha: float, extra_adds: int = 64, epilogue_abs=0.0):
    """Worst-case error of an FP32 running sum of exact products (recursive
    summation, gamma_n = n*u/(1 - n*u) with u = 2^-24) plus the epilogue's
    own roundings:

        gamma_n * |alpha| * S + 3u * E + 2u * |ref| + K * 2^-126 + 2^-149,   n = K + extra_adds

    S = sum_k |a_ik b_kj| (the oracle's ``absdot``); E = |beta*c| + |bias|
    (``epilogue_abs``, from :func:`epilogue_abs`; 0 without C and bias).
    ``extra_adds`` covers the additions a kernel makes beyond the K of the
    product (partial sums of split pieces or of K slices, the alpha
    scaling); the E term covers the rounding of beta*c and of the two
    additions that bring in beta*c and the bias, whose operands can be far
    larger than the result when they cancel; the last terms allow for FP32
    partial sums below the normal range being flushed (2^-149, the smallest
    FP32 value, keeps the bound positive).  This is a diagnostic, not the
    acceptance rule:
    an FP32-accumulating kernel stays below it on any data, while an FP16
    (or BF16) running sum exceeds it by orders of magnitude on ordinary
    data, although the acceptance rule can still pass it ("Capstone 4: a
    tensor-core GEMM", Common failures: the accumulator must not be FP16;
    "Tensor cores with WMMA", Exercise: an FP16 accumulator passed that
    page's checks)."""
    n = K + extra_adds
    gamma = n * U_FP32 / (1.0 - n * U_FP32)
    alpha = abs(float(np.float32(alpha)))
    return (gamma * alpha * np.asarray(absdot) + 3 * U_FP32 * np.asarray(epilogue_abs)
            + 2 * U_FP32 * np.abs(ref) + K * TINY_FP32 + 2.0 ** -149)


def epilogue_abs(beta: float, C=None, bias=None, rows=None, cols=None):
    """E = |beta*c_ij| + |bias_j| for :func:`accumulation_bound`: over the
    whole (M, N) C, or at entries (rows[t], cols[t]) when those are given;
    0.0 when there is neither a C term (beta == 0 or no C) nor a bias."""
    beta = float(np.float32(beta))
    e = 0.0
    if beta != 0.0 and C is not None:
        c = np.asarray(C, dtype=np.float64)
        e = np.abs(beta * (c[rows, cols] if rows is not None else c))
    if bias is not None:
        b = np.abs(np.asarray(bias, dtype=np.float64))
        e = e + (b[cols] if rows is not None else b[None, :])
    return e


def accumulation_ratio(got, ref, absdot, K: int, alpha: float, extra_adds: int = 64,
                       epilogue_abs=0.0) -> float:
    """max |got - ref| / accumulation_bound(...) over the finite entries of
    ``ref`` (NaN/Inf in ``got`` there count as infinitely far); 0 for no
    entries.  At most 1 for an FP32-accumulating kernel."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    err = np.abs(got[fin] - ref[fin])
    err = np.where(np.isfinite(err), err, np.inf)
    epi = np.broadcast_to(np.asarray(epilogue_abs, dtype=np.float64), ref.shape)[fin]
    bound = accumulation_bound(ref[fin], np.asarray(absdot)[fin], K, alpha, extra_adds, epi)
    return float(np.max(err / bound))


def worst(got, ref, absdot):
    """Diagnostics for a failure message: index of the worst element (by
    err/tol), its err and tol, and the count of failing elements."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    tol = TOL_REL * absdot + TOL_ABS
    ratio = np.where(np.isfinite(err), err / tol, np.inf)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    bad = int(np.count_nonzero(~(err <= tol)))
    return {"index": tuple(int(i) for i in idx),
            "got": float(got[idx]) if ratio.size else None,
            "want": float(ref[idx]) if ratio.size else None,
            "err": float(err[idx]) if ratio.size else None,
            "tol": float(tol[idx]) if ratio.size else None,
            "failing": bad}
