"""Seeded synthetic inputs for the FP16-input / FP32-accumulate GEMM.

This module only draws numbers: it holds none of the product's arithmetic and
imports neither the GPU library nor the oracle, so both sides can be fed the
same inputs.  Everything is drawn on the CPU with ``torch.Generator`` so the
draw does not depend on a device.

Recipe (one generator per workload, seeded, draws in the order A, B, C):
  - ``uniform``: float32 ``rand*2-1`` (i.i.d. uniform on [-1, 1)), then
    rounded to FP16 (round-to-nearest-even).
  - ``normal4``: float32 standard normal, clipped to [-4, 4], then rounded
    to FP16 (4.0 is exact in FP16).
  - ``smallint``: integers, A in [-3, 3] and B in [-2, 2], exact in FP16,
    the exact-integer fill of "Tensor cores with WMMA" (section "Why this
    program calls cuBLAS twice").
  - C, when the workload reads it (beta != 0), is float32 uniform on [-1, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str = "uniform"
    alpha: float = 1.0
    beta: float = 0.0
    c_init: Optional[str] = None
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def flop(self) -> int:
        """Floating-point operations counted as 2*M*N*K (the pages count
        GFLOP/s as 2n^3 over the time; alpha/beta work is not counted)."""
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """A and B read once (FP16), C written once (FP32), C read once more
        when beta != 0."""
        c = self.M * self.N * 4
        return 2 * self.M * self.K + 2 * self.K * self.N + c + (c if self.beta != 0 else 0)


#: The six workloads this library is measured and checked on.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("square256", 256, 256, 256, "uniform", 1.0, 0.0, None, 1000,
                 "small case; launch/latency bound"),
        Workload("square2048", 2048, 2048, 2048, "uniform", 1.0, 0.0, None, 1001,
                 "the pages' headline shape"),
        Workload("ragged1000x800x617", 1000, 800, 617, "uniform", 1.5, 0.5, "uniform", 1002,
                 "no dimension divisible by 16 or by any tile; C read with beta=0.5"),
        Workload("square8192", 8192, 8192, 8192, "normal4", 1.0, 0.0, None, 1003,
                 "compute-bound roofline shape"),
        Workload("tallskinny32768x128x4096", 32768, 128, 4096, "uniform", 1.0, 0.0, None, 1004,
                 "low reuse in N; HBM bound"),
        Workload("skinny4096x16x4096", 4096, 16, 4096, "uniform", 1.0, 0.0, None, 1005,
                 "the pages' skinny gate shape; N <= 16, an HBM stream of A"),
    )
}


def _draw(g: torch.Generator, shape, dist: str, which: str, dtype=torch.float16) -> torch.Tensor:
    if dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal4":
        x = torch.randn(shape, generator=g, dtype=torch.float32).clamp_(-4.0, 4.0)
    elif dist == "smallint":
        hi = 3 if which == "A" else 2
        x = torch.randint(-hi, hi + 1, shape, generator=g).to(torch.float32)
    elif dist == "ones":
        x = torch.ones(shape, dtype=torch.float32)
    elif dist == "zeros":
        x = torch.zeros(shape, dtype=torch.float32)
    elif dist == "adversarial":
        # FP16 edge values, every one exact in FP16 (and so in float32):
        # 10% +-65504 (the largest finite), 10% subnormals n*2^-24
        # (n = 1..1023), 10% +-2^-14 (the smallest normal), 5% zeros, the
        # rest +-(1 + f/1024)*2^e with e uniform over -14..15; signs mixed.
        # A K-term dot product stays below K*65504^2, far from FP32 overflow.
        u = torch.rand(shape, generator=g, dtype=torch.float32)
        sign = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0)
        frac = torch.randint(0, 1024, shape, generator=g).to(torch.float32)
        expo = torch.randint(-14, 16, shape, generator=g).to(torch.float32)
        sub = torch.randint(1, 1024, shape, generator=g).to(torch.float32) * 2.0 ** -24
        x = (1.0 + frac / 1024.0) * torch.exp2(expo)
        x = torch.where(u < 0.65, x, torch.where(u < 0.75, torch.full_like(x, 65504.0),
                        torch.where(u < 0.85, sub, torch.where(u < 0.95, torch.full_like(x, 2.0 ** -14),
                                                               torch.zeros_like(x)))))
        x = sign * x
        if dtype != torch.float16:
            raise ValueError("the adversarial draw is for FP16 inputs")
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.to(dtype)


def make_inputs(M: int, N: int, K: int, dist: str = "uniform", seed: int = 0,
                c_init: Optional[str] = None, dist_b: Optional[str] = None,
                dtype=torch.float16):
    """Draw (A, B, C) on the CPU: A (M,K) and B (K,N) in ``dtype`` (float16,
    or bfloat16: the same float32 draw rounded to nearest-even into the
    other format), C (M,N) fp32 or None.  ``dist_b`` overrides the
    distribution of B."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    A = _draw(g, (M, K), dist, "A", dtype)
    B = _draw(g, (K, N), dist_b or dist, "B", dtype)
    C = None
    if c_init is not None:
        if c_init == "uniform":
            C = torch.rand((M, N), generator=g, dtype=torch.float32) * 2.0 - 1.0
        elif c_init == "zeros":
            C = torch.zeros((M, N), dtype=torch.float32)
        else:
            raise ValueError(f"unknown C fill {c_init!r}")
    return A, B, C


def workload_inputs(w: Workload, dtype=torch.float16):
    return make_inputs(w.M, w.N, w.K, w.dist, w.seed, w.c_init, dtype=dtype)


def bits(t: torch.Tensor) -> np.ndarray:
    """FP16 or BF16 tensor (CPU) -> numpy uint16 array of its bit patterns."""
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("expected a float16 or bfloat16 tensor")
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def sample_entries(M: int, N: int, count: int, seed: int = 0):
    """Sampled (row, col) pairs for checking large products entry by entry:
    every corner and the last row/column edges first, then uniform draws."""
    rng = np.random.default_rng(seed)
    fixed_r = [0, 0, M - 1, M - 1, M // 2]
    fixed_c = [0, N - 1, 0, N - 1, N // 2]
    edge = min(64, max(count // 8, 1))
    er = rng.integers(0, M, edge)
    ec = rng.integers(0, N, edge)
    rows = np.concatenate([fixed_r, np.full(edge, M - 1), er,
                           rng.integers(0, M, max(count - len(fixed_r) - 2 * edge, 0))])
    cols = np.concatenate([fixed_c, ec, np.full(edge, N - 1),
                           rng.integers(0, N, max(count - len(fixed_c) - 2 * edge, 0))])
    return rows.astype(np.int64), cols.astype(np.int64)
