"""Helpers for the GPU tests: device buffers with guard margins, running the
library through its C ABI, and failure messages that name the element."""
import numpy as np
import torch

import dense_mixed_precision_amd as mp
import oracle

GUARD = 64          # guard elements before and after each device buffer
SENTINEL_F32 = np.float32(-12345.5)
SENTINEL_F16_BITS = 0x7E01  # a NaN payload nobody produces


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


class Guarded:
    """A row-major (rows, cols) view with leading dimension `ld`, carved out of
    a flat device buffer with GUARD sentinel elements on both sides, starting
    `offset` elements after an aligned base (offset=1 makes it misaligned)."""

    def __init__(self, host: torch.Tensor, ld: int = None, offset: int = 0, fill=None):
        rows, cols = host.shape
        ld = cols if ld is None else ld
        self.rows, self.cols, self.ld, self.offset = rows, cols, ld, offset
        span = (rows - 1) * ld + cols if rows > 0 and cols > 0 else 0
        total = GUARD + offset + span + GUARD
        dt = host.dtype
        if dt == torch.float16:
            flat = torch.full((total,), 0, dtype=torch.int16)
            flat.fill_(np.int16(np.uint16(SENTINEL_F16_BITS).view(np.int16)))
            flat = flat.view(torch.float16)
        else:
            flat = torch.full((total,), float(SENTINEL_F32), dtype=dt)
        self.flat_host = flat.clone()
        start = GUARD + offset
        if span:
            inner = torch.as_strided(flat, (rows, cols), (ld, 1), start)
            src = host if fill is None else torch.full_like(host, fill)
            inner.copy_(src)
            self.flat_host = flat.clone()
        self.flat = flat.to(device())
        self.start = start
        self.span = span

    def view(self):
        return torch.as_strided(self.flat, (self.rows, self.cols), (max(self.ld, 1), 1), self.start)

    def result(self) -> np.ndarray:
        flat = self.flat.cpu()
        return torch.as_strided(flat, (self.rows, self.cols), (max(self.ld, 1), 1), self.start).numpy()

    def untouched_outside_window(self) -> bool:
        """Every element outside the (rows, cols) window equals what was
        there before the call (guards and the ld-cols gap of each row)."""
        before = self.flat_host.view(torch.int16 if self.flat_host.dtype == torch.float16 else torch.int32)
        after = self.flat.cpu()
        after = after.view(torch.int16 if after.dtype == torch.float16 else torch.int32)
        mask = torch.ones(before.shape, dtype=torch.bool)
        if self.span:
            idx = torch.as_strided(torch.arange(before.numel()), (self.rows, self.cols), (max(self.ld, 1), 1), self.start)
            mask[idx.reshape(-1)] = False
        return bool(torch.equal(before[mask], after[mask]))


def run(A, B, C0, alpha, beta, config=None, lda=None, ldb=None, ldc=None,
        a_off=0, b_off=0, poison=True, stream=None):
    """Run the library on host tensors A (M,K) f16, B (K,N) f16 and C0
    (M,N) f32 or None; returns (result ndarray, guarded C)."""
    M, K = A.shape
    N = B.shape[1]
    gA = Guarded(A, ld=lda, offset=a_off)
    gB = Guarded(B, ld=ldb, offset=b_off)
    if C0 is None:
        gC = Guarded(torch.zeros((M, N), dtype=torch.float32), ld=ldc,
                     fill=float("nan") if poison else 0.0)
    else:
        gC = Guarded(C0, ld=ldc)
    mp.gemm(gA.view(), gB.view(), gC.view(), alpha, beta, config=config, stream=stream)
    torch.cuda.synchronize()
    return gC.result(), gC


def describe_failure(label, got, ref, absdot, rows=None, cols=None):
    w = oracle.worst(got, ref, absdot)
    idx = w["index"]
    if rows is not None:
        r, c = int(rows[idx[0]]), int(cols[idx[0]])
    else:
        r, c = idx if len(idx) == 2 else (idx[0], None)
    return (f"{label}: {w['failing']} element(s) outside |err| <= 1e-3*sum|ab| + 1e-5; "
            f"worst at row {r}, col {c}: got {w['got']!r}, want {w['want']!r}, "
            f"err {w['err']:.3g} > tol {w['tol']:.3g}")


def assert_close(label, got, ref, absdot, rows=None, cols=None, *, K, alpha, beta=0.0, C0=None, bias=None):
    """The acceptance rule |got - ref| <= 1e-3*S + 1e-5 on every element, and
    the accumulation diagnostic: the worst error over the bound an FP32
    running sum of K products obeys (oracle.accumulation_bound) must be at
    most 1, which an FP16 or BF16 running sum would exceed although it can
    pass the acceptance rule.  beta, C0 (the whole C before the call) and
    bias give the bound its epilogue term.  Prints the diagnostic ratio."""
    ok = oracle.tolerance_ok(got, ref, absdot)
    if not ok.all():
        raise AssertionError(describe_failure(label, got, ref, absdot, rows, cols))
    if isinstance(C0, torch.Tensor):
        C0 = C0.numpy()
    epi = oracle.epilogue_abs(beta, C0, bias, rows, cols)
    ratio = oracle.accumulation_ratio(got, ref, absdot, K, alpha, epilogue_abs=epi)
    print(f"[{label}] accumulation ratio {ratio:.3g}", flush=True)
    assert ratio <= 1.0, (f"{label}: error {ratio:.3g} times the FP32 running-sum bound "
                          f"(K = {K}): the sum is not carried in FP32")


def tile_samples(M, N, tile=128, per_tile=1, seed=0):
    """One or more random entries inside every tile x tile block, plus the
    last row and last column, so every workgroup's output is sampled."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for ti in range(0, M, tile):
        for tj in range(0, N, tile):
            h, w = min(tile, M - ti), min(tile, N - tj)
            rows.extend(ti + rng.integers(0, h, per_tile))
            cols.extend(tj + rng.integers(0, w, per_tile))
    edge = min(256, max(M, N))
    rows.extend([M - 1] * edge); cols.extend(rng.integers(0, N, edge))
    rows.extend(rng.integers(0, M, edge)); cols.extend([N - 1] * edge)
    rows.extend([0, 0, M - 1, M - 1]); cols.extend([0, N - 1, 0, N - 1])
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


def freivalds_ok(got, A, B, C0, alpha, beta, seed=0):
    """Whole-output property that holds at any size (Freivalds' check): for a
    random +-1 vector x, row i of got@x - (alpha*A@(B@x) + beta*C0@x) is a
    signed sum of the row's element errors, so if every element meets
    |err_ij| <= 1e-3*S_ij + 1e-5 (S_ij = sum_k |a_ik b_kj|) the row total is
    at most 1e-3*(|A|@(|B|@|x|))_i + 1e-5*N.  A small FP64 rounding slack is
    added.  Returns (ok, worst err/bound ratio)."""
    rng = np.random.default_rng(seed)
    N = got.shape[1]
    x = rng.choice([-1.0, 1.0], size=N)
    A64 = A.numpy().astype(np.float64)
    B64 = B.numpy().astype(np.float64)
    lhs = got.astype(np.float64) @ x
    rhs = float(np.float32(alpha)) * (A64 @ (B64 @ x))
    if C0 is not None and beta != 0:
        rhs = rhs + float(np.float32(beta)) * (C0.numpy().astype(np.float64) @ x)
    S = np.abs(A64) @ (np.abs(B64) @ np.abs(x))
    bound = 1e-3 * S + 1e-5 * N + 1e-9 * (S + np.abs(got).astype(np.float64) @ np.abs(x))
    err = np.abs(lhs - rhs)
    ok = bool(np.all(err <= bound))
    return ok, float(np.max(err / bound))


def stored(X, col_major):
    """Logical (rows, cols) host tensor -> the tensor as stored: itself
    (row-major) or its transpose, contiguous (column-major)."""
    return X.t().contiguous() if col_major else X


def run_layout(A, B, C0, alpha, beta, layout_a, layout_b, config=None, lda=None, ldb=None,
               ldc=None, a_off=0, b_off=0, poison=True, bias=None):
    """Like run(), with A and/or B stored column-major.  A (M,K) and B (K,N)
    are the logical host matrices; a column-major operand is stored as its
    transpose (leading dimension lda >= M or ldb >= K) and handed to the
    library as the transposed view, so the binding reads the storage order
    from the strides."""
    M, K = A.shape
    N = B.shape[1]
    gA = Guarded(stored(A, layout_a), ld=lda, offset=a_off)
    gB = Guarded(stored(B, layout_b), ld=ldb, offset=b_off)
    if C0 is None:
        gC = Guarded(torch.zeros((M, N), dtype=torch.float32), ld=ldc,
                     fill=float("nan") if poison else 0.0)
    else:
        gC = Guarded(C0, ld=ldc)
    a_view = gA.view().t() if layout_a else gA.view()
    b_view = gB.view().t() if layout_b else gB.view()
    bias_dev = None if bias is None else torch.as_tensor(bias, dtype=torch.float32).to(device())
    mp.gemm(a_view, b_view, gC.view(), alpha, beta, config=config, bias=bias_dev)
    torch.cuda.synchronize()
    return gC.result(), gC
