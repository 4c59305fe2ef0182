"""dense_mixed_precision_amd -- FP16-input, FP32-accumulate GEMM for gfx950.

Thin Python binding over the C ABI in ``include/mpgemm.h`` (library
``libmpgemm.so``, built in-tree by ``build.build()``) and over the
diagnostics of ``include/mpgemm_probes.h`` (``libmpgemm_probes.so``).  Every step of the
product runs in the HIP kernels; Python only marshals arguments.  There is no
CPU or library fallback: if the shared library is missing, every call raises.

Raw entry points (same names and argument order as the C ABI; pointers are
integers holding device addresses, ``stream`` a hipStream_t as an integer,
0 for the default stream):
    mpgemm_f16f32(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, stream) -> int
    mpgemm_f16f32_query(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta) -> dict
    mpgemm_f16f32_with_config(cfg, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, stream) -> int
    mpgemm_f16f32_layout(layout_a, layout_b, M, N, K, ...) -> int   (A and/or B column-major)
    mpgemm_f16f32_layout_query(layout_a, layout_b, M, N, K, ...) -> dict
    mpgemm_f16f32_layout_with_config(cfg, layout_a, layout_b, M, N, K, ...) -> int
    mpgemm_bf16f32, mpgemm_bf16f32_layout, mpgemm_bf16f32_layout_query,
    mpgemm_bf16f32_layout_with_config: the same with BF16 inputs
    mpgemm_gemm_ex(in_type, layout_a, layout_b, M, N, K, ..., alpha, beta, bias, stream) -> int
    mpgemm_gemm_ex_with_config(cfg, in_type, layout_a, layout_b, ...) -> int   (per-column bias)
    mpgemm_splitk_plan(...) -> dict, mpgemm_gemm_splitk(..., splits, workspace, bytes, stream) -> int
    mpgemm_gemm_splitk_static(..., bias, splits, stream) -> int   (no workspace, allocates nothing)
    mpgemm_num_configs(), mpgemm_config_info(id), mpgemm_strerror(code), mpgemm_version()
Diagnostics (libmpgemm_probes.so):
    mpgemm_probe_mfma_layout(shape, out, stream)
    mpgemm_probe_mfma_rate(in_type, shape, ops, ops_len, iters, workgroups, out, out_len, stream)
    mpgemm_probe_fill(mode, depth, buf, buf_bytes, footprint, shared, replicas, passes, workgroups,
                      sink, sink_len, clocks, clocks_len, stream)

Timeline build (libmpgemm_timeline.so, include/mpgemm_timeline.h), loaded
beside the product by ``load_timeline()``: mpgemm_f16f32 plus
mpgemm_timeline_entries(), mpgemm_timeline_read(out, entries) and
mpgemm_timeline_clear() -- per-workgroup stamps of the pipelined kernel.

Tensor convenience: ``gemm(A, B, C, alpha, beta)`` for torch tensors on the
GPU (A, B both float16 or both bfloat16, each row- or column-major, e.g. a
transposed view; C float32 row-major), launched on torch's current stream.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    MPGEMM_EALIGN,
    MPGEMM_ECONFIG,
    MPGEMM_EDIM,
    MPGEMM_ELAUNCH,
    MPGEMM_ELAYOUT,
    MPGEMM_ESPLIT,
    MPGEMM_ESCRATCH,
    MPGEMM_STATIC_SCRATCH_BYTES,
    MPGEMM_ETYPE,
    MPGEMM_EWORKSPACE,
    MPGEMM_ELD,
    MPGEMM_ENULL,
    MPGEMM_OK,
    MPGEMM_COL_MAJOR,
    MPGEMM_IN_BF16,
    MPGEMM_IN_F16,
    MPGEMM_ROW_MAJOR,
    MPGEMM_FILL_LDS16,
    MPGEMM_FILL_REG16,
    MPGEMM_FILL_REG4,
    CANDIDATES_PATH,
    TIMELINE_PATH,
    TIMELINE_SLOTS,
    MpgemmError,
    config_fields,
    gemm,
    lib_path,
    load,
    load_probes,
    load_timeline,
    mpgemm_config_info,
    mpgemm_f16f32,
    mpgemm_f16f32_query,
    mpgemm_f16f32_with_config,
    mpgemm_f16f32_layout,
    mpgemm_f16f32_layout_query,
    mpgemm_f16f32_layout_with_config,
    mpgemm_bf16f32,
    mpgemm_bf16f32_layout,
    mpgemm_bf16f32_layout_query,
    mpgemm_bf16f32_layout_with_config,
    mpgemm_gemm_ex,
    mpgemm_gemm_ex_with_config,
    mpgemm_splitk_plan,
    mpgemm_gemm_splitk,
    mpgemm_gemm_splitk_static,
    gemm_splitk,
    splitk_plan_for,
    mpgemm_num_configs,
    mpgemm_probe_mfma_layout,
    mpgemm_probe_mfma_rate,
    mpgemm_probe_fill,
    mpgemm_strerror,
    mpgemm_version,
    query_for,
)
