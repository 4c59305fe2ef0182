"""ctypes binding for libmpgemm.so and the diagnostics libraries
libmpgemm_probes.so and libmpgemm_timeline.so (argument marshalling only:
every step of the product runs in the HIP library)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmpgemm.so")
_PROBES_PATH = os.path.join(_HERE, "libmpgemm_probes.so")
#: the product library plus the sweep-only tile shapes (built on request)
CANDIDATES_PATH = os.path.join(_HERE, "libmpgemm_candidates.so")
#: the product library with the per-workgroup timeline (include/mpgemm_timeline.h)
TIMELINE_PATH = os.path.join(_HERE, "libmpgemm_timeline.so")
#: uint64 stamps per workgroup record of the timeline build
TIMELINE_SLOTS = 48

MPGEMM_OK = 0
MPGEMM_EDIM = -1
MPGEMM_ELD = -2
MPGEMM_ENULL = -3
MPGEMM_ELAUNCH = -4
MPGEMM_ECONFIG = -5
MPGEMM_EALIGN = -6
MPGEMM_ELAYOUT = -7
MPGEMM_ETYPE = -8
MPGEMM_EWORKSPACE = -9
MPGEMM_ESPLIT = -10
MPGEMM_ESCRATCH = -11
#: bytes of the static split-K scratch of mpgemm_gemm_splitk_static
MPGEMM_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024

MPGEMM_ROW_MAJOR = 0
MPGEMM_COL_MAJOR = 1

MPGEMM_IN_F16 = 0
MPGEMM_IN_BF16 = 1


class MpgemmConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "id", "kind", "bm", "bn", "bk", "waves_m", "waves_n", "wave_m", "wave_n",
        "mfma_m", "mfma_n", "mfma_k", "vec_a", "vec_b", "stages", "threads", "lds_bytes")] + [
        ("grid", ctypes.c_int64), ("layout_a", ctypes.c_int32), ("layout_b", ctypes.c_int32),
        ("in_type", ctypes.c_int32), ("k_groups", ctypes.c_int32), ("k_order", ctypes.c_int32),
        ("c_stores", ctypes.c_int32)]


config_fields = [f[0] for f in MpgemmConfig._fields_]
KIND_NAMES = {1: "direct", 2: "scale", 3: "none", 4: "pipe", 5: "narrow"}

MPGEMM_FILL_LDS16 = 0
MPGEMM_FILL_REG16 = 1
MPGEMM_FILL_REG4 = 2


class MpgemmError(RuntimeError):
    def __init__(self, code: int, where: str = "mpgemm"):
        self.code = code
        super().__init__(f"{where}: error {code}: {mpgemm_strerror(code)}")


_lib = None
_lib_path = None
_probes = None


def lib_path() -> str:
    return _lib_path or _LIB_PATH


def load(path: str | None = None):
    """Load the in-tree libmpgemm.so (or, once, before anything else is
    loaded, the library at `path`: the candidates build for tile sweeps).
    Raises if it has not been built; there is no fallback path."""
    global _lib, _lib_path
    if _lib is not None:
        if path is not None and os.path.abspath(path) != _lib_path:
            raise RuntimeError(f"{_lib_path} is already loaded; cannot switch to {path}")
        return _lib
    path = os.path.abspath(path or _LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m dense_mixed_precision_amd.build [--candidates]` (no fallback path exists)")
    lib = ctypes.CDLL(path)
    i64, f32, vp, i32 = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    gemm_args = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, f32]
    lib.mpgemm_f16f32.argtypes = gemm_args + [vp]
    lib.mpgemm_f16f32.restype = i32
    lib.mpgemm_f16f32_query.argtypes = gemm_args + [ctypes.POINTER(MpgemmConfig)]
    lib.mpgemm_f16f32_query.restype = i32
    lib.mpgemm_f16f32_with_config.argtypes = [i32] + gemm_args + [vp]
    lib.mpgemm_f16f32_with_config.restype = i32
    lib.mpgemm_f16f32_layout.argtypes = [i32, i32] + gemm_args + [vp]
    lib.mpgemm_f16f32_layout.restype = i32
    lib.mpgemm_f16f32_layout_query.argtypes = [i32, i32] + gemm_args + [ctypes.POINTER(MpgemmConfig)]
    lib.mpgemm_f16f32_layout_query.restype = i32
    lib.mpgemm_f16f32_layout_with_config.argtypes = [i32, i32, i32] + gemm_args + [vp]
    lib.mpgemm_f16f32_layout_with_config.restype = i32
    for dt in ("bf16",):
        getattr(lib, f"mpgemm_{dt}f32").argtypes = gemm_args + [vp]
        getattr(lib, f"mpgemm_{dt}f32").restype = i32
        getattr(lib, f"mpgemm_{dt}f32_layout").argtypes = [i32, i32] + gemm_args + [vp]
        getattr(lib, f"mpgemm_{dt}f32_layout").restype = i32
        getattr(lib, f"mpgemm_{dt}f32_layout_query").argtypes = [i32, i32] + gemm_args + [
            ctypes.POINTER(MpgemmConfig)]
        getattr(lib, f"mpgemm_{dt}f32_layout_query").restype = i32
        getattr(lib, f"mpgemm_{dt}f32_layout_with_config").argtypes = [i32, i32, i32] + gemm_args + [vp]
        getattr(lib, f"mpgemm_{dt}f32_layout_with_config").restype = i32
    lib.mpgemm_gemm_ex.argtypes = [i32, i32, i32] + gemm_args + [vp, vp]
    lib.mpgemm_gemm_ex.restype = i32
    lib.mpgemm_gemm_ex_with_config.argtypes = [i32, i32, i32, i32] + gemm_args + [vp, vp]
    lib.mpgemm_gemm_ex_with_config.restype = i32
    lib.mpgemm_splitk_plan.argtypes = [i32, i32, i32, i64, i64, i64, vp, i64, vp, i64, i32,
                                       ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(i64),
                                       ctypes.POINTER(ctypes.c_int32)]
    lib.mpgemm_splitk_plan.restype = i32
    lib.mpgemm_gemm_splitk.argtypes = [i32, i32, i32] + gemm_args + [vp, i32, vp, i64, vp]
    lib.mpgemm_gemm_splitk.restype = i32
    lib.mpgemm_gemm_splitk_static.argtypes = [i32, i32, i32] + gemm_args + [vp, i32, vp]
    lib.mpgemm_gemm_splitk_static.restype = i32
    lib.mpgemm_num_configs.argtypes = []
    lib.mpgemm_num_configs.restype = i32
    lib.mpgemm_config_info.argtypes = [i32, ctypes.POINTER(MpgemmConfig)]
    lib.mpgemm_config_info.restype = i32
    lib.mpgemm_strerror.argtypes = [i32]
    lib.mpgemm_strerror.restype = ctypes.c_char_p
    lib.mpgemm_version.argtypes = []
    lib.mpgemm_version.restype = ctypes.c_char_p
    _lib = lib
    _lib_path = path
    return lib


def load_probes():
    """Load the in-tree diagnostics library libmpgemm_probes.so."""
    global _probes
    if _probes is not None:
        return _probes
    if not os.path.exists(_PROBES_PATH):
        raise RuntimeError(f"{_PROBES_PATH} is not built; run `python -m dense_mixed_precision_amd.build`")
    lib = ctypes.CDLL(_PROBES_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.mpgemm_probe_mfma_layout.argtypes = [i32, vp, vp]
    lib.mpgemm_probe_mfma_layout.restype = i32
    lib.mpgemm_probe_mfma_rate.argtypes = [i32, i32, vp, i64, i64, i32, vp, i64, vp]
    lib.mpgemm_probe_mfma_rate.restype = i32
    lib.mpgemm_probe_fill.argtypes = [i32, i32, vp, i64, i64, i32, i32, i64, i32, vp, i64, vp, i64, vp]
    lib.mpgemm_probe_fill.restype = i32
    _probes = lib
    return lib


_timeline = None


def load_timeline():
    """Load the timeline build (libmpgemm_timeline.so) on its own, beside the
    product library: a ctypes handle with mpgemm_f16f32 and the three
    mpgemm_timeline_* entry points typed."""
    global _timeline
    if _timeline is not None:
        return _timeline
    if not os.path.exists(TIMELINE_PATH):
        raise RuntimeError(f"{TIMELINE_PATH} is not built; run `python -m dense_mixed_precision_amd.build`")
    lib = ctypes.CDLL(TIMELINE_PATH)
    i64, vp, i32, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.mpgemm_f16f32.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, f32, vp]
    lib.mpgemm_f16f32.restype = i32
    lib.mpgemm_timeline_entries.argtypes = []
    lib.mpgemm_timeline_entries.restype = i64
    lib.mpgemm_timeline_read.argtypes = [vp, i64]
    lib.mpgemm_timeline_read.restype = i32
    lib.mpgemm_timeline_clear.argtypes = []
    lib.mpgemm_timeline_clear.restype = i32
    _timeline = lib
    return lib


def _cfg_dict(c: MpgemmConfig) -> dict:
    d = {name: int(getattr(c, name)) for name in config_fields}
    d["kind_name"] = KIND_NAMES.get(d["kind"], "?")
    return d


# ---- raw entry points (same names as the C ABI) ----------------------------

def mpgemm_f16f32(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, stream=0) -> int:
    return int(load().mpgemm_f16f32(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, stream))


def mpgemm_f16f32_query(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta) -> dict:
    out = MpgemmConfig()
    rc = load().mpgemm_f16f32_query(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                                    ctypes.byref(out))
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, "mpgemm_f16f32_query")
    return _cfg_dict(out)


def mpgemm_f16f32_with_config(config_id, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                              stream=0) -> int:
    return int(load().mpgemm_f16f32_with_config(config_id, M, N, K, A, lda, B, ldb, C, ldc,
                                                 alpha, beta, stream))


def mpgemm_f16f32_layout(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                         stream=0) -> int:
    return int(load().mpgemm_f16f32_layout(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc,
                                           alpha, beta, stream))


def mpgemm_f16f32_layout_query(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                               beta) -> dict:
    out = MpgemmConfig()
    rc = load().mpgemm_f16f32_layout_query(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc,
                                           alpha, beta, ctypes.byref(out))
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, "mpgemm_f16f32_layout_query")
    return _cfg_dict(out)


def mpgemm_f16f32_layout_with_config(config_id, layout_a, layout_b, M, N, K, A, lda, B, ldb, C,
                                     ldc, alpha, beta, stream=0) -> int:
    return int(load().mpgemm_f16f32_layout_with_config(config_id, layout_a, layout_b, M, N, K, A,
                                                       lda, B, ldb, C, ldc, alpha, beta, stream))


def mpgemm_bf16f32(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, stream=0) -> int:
    return int(load().mpgemm_bf16f32(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, stream))


def mpgemm_bf16f32_layout(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                          stream=0) -> int:
    return int(load().mpgemm_bf16f32_layout(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc,
                                            alpha, beta, stream))


def mpgemm_bf16f32_layout_query(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                                beta) -> dict:
    out = MpgemmConfig()
    rc = load().mpgemm_bf16f32_layout_query(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc,
                                            alpha, beta, ctypes.byref(out))
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, "mpgemm_bf16f32_layout_query")
    return _cfg_dict(out)


def mpgemm_bf16f32_layout_with_config(config_id, layout_a, layout_b, M, N, K, A, lda, B, ldb, C,
                                      ldc, alpha, beta, stream=0) -> int:
    return int(load().mpgemm_bf16f32_layout_with_config(config_id, layout_a, layout_b, M, N, K, A,
                                                        lda, B, ldb, C, ldc, alpha, beta, stream))


def mpgemm_gemm_ex(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                   bias=0, stream=0) -> int:
    return int(load().mpgemm_gemm_ex(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc,
                                     alpha, beta, bias, stream))


def mpgemm_gemm_ex_with_config(config_id, in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb,
                               C, ldc, alpha, beta, bias=0, stream=0) -> int:
    return int(load().mpgemm_gemm_ex_with_config(config_id, in_type, layout_a, layout_b, M, N, K,
                                                 A, lda, B, ldb, C, ldc, alpha, beta, bias, stream))


def mpgemm_splitk_plan(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb,
                       splits_requested=0) -> dict:
    """The split-K plan: {"splits", "workspace_bytes", "config_id"}."""
    sp, ws, cid = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
    rc = load().mpgemm_splitk_plan(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb,
                                   splits_requested, ctypes.byref(sp), ctypes.byref(ws),
                                   ctypes.byref(cid))
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, "mpgemm_splitk_plan")
    return {"splits": int(sp.value), "workspace_bytes": int(ws.value), "config_id": int(cid.value)}


def mpgemm_gemm_splitk(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                       bias=0, splits_requested=0, workspace=0, workspace_bytes=0, stream=0) -> int:
    return int(load().mpgemm_gemm_splitk(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C,
                                         ldc, alpha, beta, bias, splits_requested, workspace,
                                         workspace_bytes, stream))


def mpgemm_gemm_splitk_static(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                              beta, bias=0, splits_requested=0, stream=0) -> int:
    return int(load().mpgemm_gemm_splitk_static(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C,
                                                ldc, alpha, beta, bias, splits_requested, stream))


def mpgemm_num_configs() -> int:
    return int(load().mpgemm_num_configs())


def mpgemm_config_info(config_id: int) -> dict:
    out = MpgemmConfig()
    rc = load().mpgemm_config_info(config_id, ctypes.byref(out))
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, "mpgemm_config_info")
    return _cfg_dict(out)


def mpgemm_probe_mfma_layout(shape: int, out: int, stream=0) -> int:
    return int(load_probes().mpgemm_probe_mfma_layout(shape, out, stream))


def mpgemm_probe_mfma_rate(in_type: int, shape: int, ops: int, ops_len: int, iters: int, workgroups: int,
                           out: int, out_len: int, stream=0) -> int:
    return int(load_probes().mpgemm_probe_mfma_rate(in_type, shape, ops, ops_len, iters, workgroups, out,
                                                    out_len, stream))


def mpgemm_probe_fill(mode: int, depth: int, buf: int, buf_bytes: int, footprint: int, shared: int,
                      replicas: int, passes: int, workgroups: int, sink: int, sink_len: int, clocks: int = 0,
                      clocks_len: int = 0, stream=0) -> int:
    return int(load_probes().mpgemm_probe_fill(mode, depth, buf, buf_bytes, footprint, shared, replicas,
                                               passes, workgroups, sink, sink_len, clocks, clocks_len, stream))


def mpgemm_strerror(code: int) -> str:
    return load().mpgemm_strerror(code).decode()


def mpgemm_version() -> str:
    return load().mpgemm_version().decode()


# ---- torch tensor convenience ----------------------------------------------

def _check_tensor(t, name, dtype, allow_col_major=False):
    """Validate a 2-D GPU tensor; returns (layout, leading dimension).

    Row-major: unit stride along dimension 1, ld = stride(0).  Column-major
    (A and B only): unit stride along dimension 0, ld = stride(1).  An
    extent-1 dimension's stride is ignored."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    rows, cols = t.shape
    if cols <= 1 or t.stride(1) == 1:
        if rows <= 1:
            return MPGEMM_ROW_MAJOR, max(cols, 1)
        # rows that share memory (a broadcast or overlapping view) would be
        # read wrongly or, for C, written out of bounds: refuse them
        if t.stride(0) < max(cols, 1):
            raise ValueError(f"{name}: its rows overlap (row stride {t.stride(0)} < {cols} columns)")
        return MPGEMM_ROW_MAJOR, t.stride(0)
    if allow_col_major and (rows <= 1 or t.stride(0) == 1):
        # here cols > 1: the columns are the stored rows
        if t.stride(1) < max(rows, 1):
            raise ValueError(f"{name}: its columns overlap (column stride {t.stride(1)} < {rows} rows)")
        return MPGEMM_COL_MAJOR, t.stride(1)
    raise ValueError(f"{name} must have unit stride along one dimension"
                     + ("" if allow_col_major else " (row-major)"))


def _args(A, B, C):
    import torch
    dt = A.dtype if isinstance(A, torch.Tensor) and A.dtype == torch.bfloat16 else torch.float16
    la, lda = _check_tensor(A, "A", dt, allow_col_major=True)
    lb, ldb = _check_tensor(B, "B", dt, allow_col_major=True)
    _, ldc = _check_tensor(C, "C", torch.float32)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    return M, N, K, la, lda, lb, ldb, ldc


def _in_type(A):
    import torch
    return MPGEMM_IN_BF16 if A.dtype == torch.bfloat16 else MPGEMM_IN_F16


def _bias_ptr(bias, N):
    import torch
    if bias is None:
        return 0
    if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32 or not bias.is_cuda:
        raise TypeError("bias must be a float32 tensor on the GPU")
    if bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1):
        raise ValueError(f"bias must be a contiguous vector of N = {N} values")
    return bias.data_ptr()


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, config: int | None = None, stream=None,
         bias=None):
    """C <- alpha*A@B + beta*C (+ bias[j]) in place on the GPU; returns C.

    A (M x K) and B (K x N): both float16 or both bfloat16, each row-major or
    column-major (e.g. the transpose view of a row-major tensor); the storage
    order is read from the strides.  C must be float32 row-major.  ``bias``:
    optional float32 vector of N values added to every row.
    ``stream``: a torch.cuda.Stream or raw handle (default: current stream).
    ``config``: force a table entry (tests and sweeps)."""
    import torch
    M, N, K, la, lda, lb, ldb, ldc = _args(A, B, C)
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    in_type = _in_type(A)
    bf16 = in_type == MPGEMM_IN_BF16
    if bias is not None:
        bp = _bias_ptr(bias, N)
        if config is None:
            rc = mpgemm_gemm_ex(in_type, la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                C.data_ptr(), ldc, float(alpha), float(beta), bp, handle)
        else:
            rc = mpgemm_gemm_ex_with_config(int(config), in_type, la, lb, M, N, K, A.data_ptr(), lda,
                                            B.data_ptr(), ldb, C.data_ptr(), ldc, float(alpha),
                                            float(beta), bp, handle)
        if rc != MPGEMM_OK:
            raise MpgemmError(rc, "mpgemm_gemm_ex" if config is None else f"config {config}")
        return C
    if config is None and not bf16 and (la, lb) == (MPGEMM_ROW_MAJOR, MPGEMM_ROW_MAJOR):
        rc = mpgemm_f16f32(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                           float(alpha), float(beta), handle)
        if rc != MPGEMM_OK:
            raise MpgemmError(rc, "mpgemm_f16f32")
        return C
    if config is None:
        fn = mpgemm_bf16f32_layout if bf16 else mpgemm_f16f32_layout
        rc = fn(la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                float(alpha), float(beta), handle)
    else:
        fn = mpgemm_bf16f32_layout_with_config if bf16 else mpgemm_f16f32_layout_with_config
        rc = fn(int(config), la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(),
                ldc, float(alpha), float(beta), handle)
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, fn.__name__ if config is None else f"config {config}")
    return C


def query_for(A, B, C, alpha: float = 1.0, beta: float = 0.0) -> dict:
    """The factory's choice for these tensors (no launch)."""
    M, N, K, la, lda, lb, ldb, ldc = _args(A, B, C)
    fn = mpgemm_bf16f32_layout_query if _in_type(A) == MPGEMM_IN_BF16 else mpgemm_f16f32_layout_query
    return fn(la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
              float(alpha), float(beta))


def splitk_plan_for(A, B, C, splits: int = 0) -> dict:
    """The split-K plan for these tensors (no launch)."""
    M, N, K, la, lda, lb, ldb, ldc = _args(A, B, C)
    return mpgemm_splitk_plan(_in_type(A), la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                              int(splits))


def gemm_splitk(A, B, C, alpha: float = 1.0, beta: float = 0.0, bias=None, splits: int = 0,
                workspace=None, stream=None):
    """Split-K form of :func:`gemm`.  ``splits`` 0 lets the library decide.
    ``workspace``: a contiguous float32 tensor on C's GPU of at least the
    planned size; when None, one is allocated here (by torch, on the
    caller's side of the C ABI) for this call."""
    import torch
    M, N, K, la, lda, lb, ldb, ldc = _args(A, B, C)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.float32 or not workspace.is_cuda:
            raise TypeError("workspace must be a float32 tensor on the GPU")
        if workspace.device != C.device:
            raise ValueError(f"workspace is on {workspace.device}, C on {C.device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous (the kernels write it as one flat array)")
    plan = mpgemm_splitk_plan(_in_type(A), la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                              int(splits))
    if workspace is None and plan["workspace_bytes"] > 0:
        workspace = torch.empty(plan["workspace_bytes"] // 4, dtype=torch.float32, device=C.device)
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    rc = mpgemm_gemm_splitk(_in_type(A), la, lb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                            C.data_ptr(), ldc, float(alpha), float(beta), _bias_ptr(bias, N),
                            int(splits), ws_ptr, ws_bytes, handle)
    if rc != MPGEMM_OK:
        raise MpgemmError(rc, "mpgemm_gemm_splitk")
    return C
