"""Exact rational arithmetic for pinning the oracle on tiny inputs.

Independent of the oracle: FP16 values are decoded with numpy's own float16
conversion (a library routine) and summed as exact rationals
(``fractions.Fraction``), so the result is the true value of
``alpha * sum_k a_ik b_kj + beta * c_ij`` with no rounding at all.
"""
from fractions import Fraction

import numpy as np


def f16_exact(bits_2d):
    """FP16 bit patterns -> nested lists of exact Fractions (via numpy)."""
    vals = np.asarray(bits_2d, dtype=np.uint16).view(np.float16).astype(np.float64)
    return [[Fraction(float(v)) for v in row] for row in vals]


def bf16_exact(bits_2d):
    """BF16 bit patterns -> nested lists of exact Fractions (via torch's own
    bfloat16 -> float64 conversion, a library routine)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(bits_2d, dtype=np.uint16)).view(np.int16))
    vals = t.view(torch.bfloat16).to(torch.float64).numpy()
    return [[Fraction(float(v)) for v in row] for row in vals]


def exact_gemm(A_bits, B_bits, C=None, alpha=1.0, beta=0.0, in_type="f16", bias=None):
    """Exact result and exact sum|a*b| as float64 arrays (rounded once at the
    end, to nearest) plus the exact Fractions for callers that need them."""
    decode = bf16_exact if in_type == "bf16" else f16_exact
    A = decode(A_bits)
    B = decode(B_bits)
    M, K = len(A), (len(A[0]) if A else 0)
    N = len(B[0]) if B else np.asarray(B_bits).shape[1]
    fa = Fraction(float(np.float32(alpha)))
    fb = Fraction(float(np.float32(beta)))
    ref = np.empty((M, N))
    absdot = np.empty((M, N))
    exact = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                p = A[i][k] * B[k][j]
                s += p
                sa += abs(p)
            r = fa * s
            if fb != 0:
                r += fb * Fraction(float(C[i, j]))
            if bias is not None:
                r += Fraction(float(bias[j]))
            exact[i][j] = r
            ref[i, j] = float(r)
            absdot[i, j] = float(sa)
    return ref, absdot, exact


def fp64_sum_bound(K, alpha, beta, absdot, C=None, bias=None):
    """Worst-case rounding of an FP64 ascending sum of K exact products plus
    the alpha/beta (and bias) combination:
    (K + 5) * 2^-53 * (|alpha|*S + |beta*c| + |bias|)."""
    u = 2.0 ** -53
    extra = 0.0 if (C is None or beta == 0) else np.abs(float(np.float32(beta)) * C.astype(np.float64))
    if bias is not None:
        extra = extra + np.abs(np.asarray(bias, dtype=np.float64))[None, :]
    return (K + 5) * u * (abs(float(np.float32(alpha))) * absdot + extra) + 1e-300
