/*
 * mpgemm.h -- C ABI of the FP16-input, FP32-accumulate GEMM for gfx950
 * (AMD Instinct MI355X).
 *
 * The operation (the mixed-precision contract of "Capstone 4: a tensor-core
 * GEMM", sections "Capability" and "Minimal model": FP16 inputs, an FP32
 * running sum and an FP32 result, correct when no tile divides the matrix):
 *
 *     C[i][j] <- alpha * sum_{k<K} A[i][k] * B[k][j] + beta * C[i][j]
 *                for 0 <= i < M, 0 <= j < N
 *
 * Layouts.  In mpgemm_f16f32 all three matrices are row-major and live in
 * device memory:
 *     A[i][k] at A[i*lda + k]   (M x K, FP16 bit patterns, lda >= max(1,K))
 *     B[k][j] at B[k*ldb + j]   (K x N, FP16 bit patterns, ldb >= max(1,N))
 *     C[i][j] at C[i*ldc + j]   (M x N, IEEE binary32,     ldc >= max(1,N))
 * The *_layout entry points also take A and/or B column-major (see
 * mpgemm_f16f32_layout); C is always row-major.
 * Leading dimensions count elements, not bytes.  Any M, N, K >= 0 is
 * accepted; no padding is needed and none is done.  A and B must be 2-byte
 * aligned and C 4-byte aligned.  A and B are read with 16-byte vector loads
 * whatever their alignment (gfx950 under ROCm serves unaligned vector loads),
 * so odd leading dimensions and offset pointers take the same fast path.
 *
 * Arithmetic.  Products of FP16 values are exact in FP32 and are summed in
 * FP32 by the matrix cores; alpha and beta are applied in FP32 at the end.
 * When beta == 0, C is written without being read (it may hold NaN).  When
 * alpha == 0 or K == 0, A and B are not read and C <- beta*C.  Elements of C
 * outside the M x N window (columns N..ldc-1) are never touched.
 *
 * Ownership and concurrency.  The caller owns every buffer.  The library
 * allocates nothing, frees nothing, keeps no per-call state and never
 * synchronizes: work is enqueued on `stream` (a hipStream_t passed as
 * void*; NULL is the default stream) and is complete when the stream is.
 * Entry points may be called from several host threads at once.  Calls
 * whose output regions overlap race like any two kernels writing the same
 * memory.
 *
 * Errors.  Every entry point returns 0 on success or a negative
 * MPGEMM_E* code.  Argument errors are detected on the host before any HIP
 * call, so nothing is enqueued.  MPGEMM_ELAUNCH reports the HIP error that
 * the launch itself returned.
 */
#ifndef MPGEMM_H
#define MPGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MPGEMM_OK 0
#define MPGEMM_EDIM (-1)       /* M, N or K negative                              */
#define MPGEMM_ELD (-2)        /* a leading dimension below its stored row length  */
#define MPGEMM_ENULL (-3)      /* NULL pointer for an operand that must be read   */
#define MPGEMM_ELAUNCH (-4)    /* the HIP launch failed                           */
#define MPGEMM_ECONFIG (-5)    /* unknown config id, or it cannot run these args  */
#define MPGEMM_EALIGN (-6)     /* A/B not 2-byte aligned, C or bias not 4-byte    */
#define MPGEMM_ELAYOUT (-7)    /* a layout argument is not one of MPGEMM_*_MAJOR  */
#define MPGEMM_ETYPE (-8)      /* an input type is not one of MPGEMM_IN_*         */
#define MPGEMM_EWORKSPACE (-9) /* split-K workspace smaller than planned          */
#define MPGEMM_ESPLIT (-10)    /* negative split count requested                  */
#define MPGEMM_ESCRATCH (-11)  /* split-K plan larger than the static scratch     */

/* Storage order of A or B (C is always row-major). */
#define MPGEMM_ROW_MAJOR 0
#define MPGEMM_COL_MAJOR 1

/* Input format of A and B (the accumulator and C are always FP32). */
#define MPGEMM_IN_F16 0        /* IEEE binary16                                   */
#define MPGEMM_IN_BF16 1       /* bfloat16                                        */

/* Kinds of kernel a config can name (0 is not used). */
#define MPGEMM_KIND_DIRECT 1   /* operands straight from memory; any size/stride  */
#define MPGEMM_KIND_SCALE 2    /* C <- beta*C only (alpha == 0 or K == 0)         */
#define MPGEMM_KIND_NONE 3     /* nothing to do (M == 0 or N == 0)                */
#define MPGEMM_KIND_PIPE 4     /* LDS ring filled by direct-to-LDS copies; operands
                                  stored along M or N read with the transposing
                                  LDS load; the fast path                         */
#define MPGEMM_KIND_NARROW 5   /* N <= 16, A row-major: 16 rows of C per workgroup,
                                  8 waves splitting K, operands straight from
                                  memory into registers, partial tiles summed in
                                  LDS                                             */

/* One entry of the kernel-config table, as reported by the factory. */
typedef struct mpgemm_config {
    int32_t id;          /* index in the table (see mpgemm_num_configs)          */
    int32_t kind;        /* MPGEMM_KIND_*                                         */
    int32_t bm, bn, bk;  /* block tile: rows of C, columns of C, K per LDS stage  */
    int32_t waves_m;     /* waves along M in a workgroup                          */
    int32_t waves_n;     /* waves along N                                         */
    int32_t wave_m;      /* rows of C per wave                                    */
    int32_t wave_n;      /* columns of C per wave                                 */
    int32_t mfma_m, mfma_n, mfma_k; /* matrix instruction: 32x32x16 or 16x16x32   */
    int32_t vec_a;       /* 16-bit elements per global load of A: 8 for the tiled
                            kernels (16-byte loads at any 2-byte alignment), 1
                            for the direct kernel (element loads)                 */
    int32_t vec_b;       /* the same for B                                        */
    int32_t stages;      /* LDS buffers in flight                                 */
    int32_t threads;     /* threads per workgroup                                 */
    int32_t lds_bytes;   /* LDS per workgroup                                     */
    int64_t grid;        /* workgroups for the queried shape (0 in the table)     */
    int32_t layout_a;    /* storage order of A the entry reads (MPGEMM_*_MAJOR)   */
    int32_t layout_b;    /* storage order of B; the direct and scale kernels take
                            any order and report the one they were asked for.
                            A one-column row-major B with ldb == 1 (K
                            consecutive values) is read, and reported, as
                            column-major: the same bytes                        */
    int32_t in_type;     /* input format the entry reads (MPGEMM_IN_*)            */
    int32_t k_groups;    /* wave groups sharing each LDS tile, each taking its own
                            k-steps over the whole block; threads =
                            64 * waves_m * waves_n * k_groups                     */
    int32_t k_order;     /* order of K tiles: 0 ascending in every workgroup; D >= 2
                            staggered: the workgroup at tile row tm, tile column
                            tn starts at K tile (tm + tn) mod min(D, K tiles)
                            and wraps round (its sum over K is taken in another
                            order, so its rounding differs from the ascending
                            entry's)                                            */
    int32_t c_stores;    /* cache policy of the stores of C: for a queried call
                            1 non-temporal, 0 plain; in the table 1 or 0 for
                            an entry built with that policy only, 2 for one
                            built with both (256x256 tiles: plain when more
                            than 176 of them write their C in one round at
                            K < 2048, or when the rows of C start mid-line)  */
} mpgemm_config;

/*
 * The GEMM.  Picks a kernel config for the shape, alignment and scalars
 * (the same choice mpgemm_f16f32_query reports) and enqueues it on
 * `stream`.  Returns MPGEMM_OK or a negative code; see the file header for
 * the arguments, layouts and semantics.
 */
int mpgemm_f16f32(int64_t M, int64_t N, int64_t K,
                  const uint16_t *A, int64_t lda,
                  const uint16_t *B, int64_t ldb,
                  float *C, int64_t ldc,
                  float alpha, float beta,
                  void *stream);

/*
 * The factory's choice for these arguments, without launching anything and
 * without any HIP call (pointers are only inspected for alignment and NULL).
 * Fills *out and returns MPGEMM_OK, or returns the error mpgemm_f16f32
 * would return.  `out` is caller-owned host memory.
 */
int mpgemm_f16f32_query(int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb,
                        const float *C, int64_t ldc,
                        float alpha, float beta,
                        mpgemm_config *out);

/*
 * The GEMM forced onto table entry `config_id` (for tests and tile sweeps).
 * Same arguments and semantics as mpgemm_f16f32.  Returns MPGEMM_ECONFIG if
 * the id is unknown or the entry cannot run these arguments (for example an
 * entry for another storage order or input format, or the scale-only entry
 * with K > 0).
 */
int mpgemm_f16f32_with_config(int config_id,
                              int64_t M, int64_t N, int64_t K,
                              const uint16_t *A, int64_t lda,
                              const uint16_t *B, int64_t ldb,
                              float *C, int64_t ldc,
                              float alpha, float beta,
                              void *stream);

/*
 * The GEMM with A and/or B stored column-major, as the operands of the
 * independent gate of "Capstone 4: a tensor-core GEMM" (section
 * "Independent gate": A row-major, B column-major, C row-major):
 *     layout_a == MPGEMM_ROW_MAJOR: A[i][k] at A[i*lda + k], lda >= max(1,K)
 *     layout_a == MPGEMM_COL_MAJOR: A[i][k] at A[k*lda + i], lda >= max(1,M)
 *     layout_b == MPGEMM_ROW_MAJOR: B[k][j] at B[k*ldb + j], ldb >= max(1,N)
 *     layout_b == MPGEMM_COL_MAJOR: B[k][j] at B[j*ldb + k], ldb >= max(1,K)
 * Everything else (C, alpha, beta, alignment, errors, ownership) is as for
 * mpgemm_f16f32, which is this call with (MPGEMM_ROW_MAJOR, MPGEMM_ROW_MAJOR).
 * A layout value other than the two above returns MPGEMM_ELAYOUT.
 */
int mpgemm_f16f32_layout(int layout_a, int layout_b,
                         int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb,
                         float *C, int64_t ldc,
                         float alpha, float beta,
                         void *stream);

/* The factory's choice for mpgemm_f16f32_layout (no launch, no HIP call). */
int mpgemm_f16f32_layout_query(int layout_a, int layout_b,
                               int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb,
                               const float *C, int64_t ldc,
                               float alpha, float beta,
                               mpgemm_config *out);

/*
 * mpgemm_f16f32_layout forced onto table entry `config_id`.  MPGEMM_ECONFIG
 * if the entry was compiled for other storage orders (its layout_a and
 * layout_b fields) or cannot run these arguments.
 */
int mpgemm_f16f32_layout_with_config(int config_id, int layout_a, int layout_b,
                                     int64_t M, int64_t N, int64_t K,
                                     const uint16_t *A, int64_t lda,
                                     const uint16_t *B, int64_t ldb,
                                     float *C, int64_t ldc,
                                     float alpha, float beta,
                                     void *stream);

/*
 * The same GEMM with BF16 inputs: A and B hold bfloat16 bit patterns (the
 * other 16-bit tensor-core input type listed in "Tensor cores with WMMA",
 * section "A warp owns a tile, and no thread owns an element").  Products
 * of BF16 values are exact in FP32 and summed in FP32, as for FP16.  Every
 * other argument, layout rule, error and the semantics are those of the
 * FP16 entry point of the same form; mpgemm_bf16f32 takes row-major A and B.
 */
int mpgemm_bf16f32(int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb,
                   float *C, int64_t ldc,
                   float alpha, float beta,
                   void *stream);

int mpgemm_bf16f32_layout(int layout_a, int layout_b,
                          int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda,
                          const uint16_t *B, int64_t ldb,
                          float *C, int64_t ldc,
                          float alpha, float beta,
                          void *stream);

int mpgemm_bf16f32_layout_query(int layout_a, int layout_b,
                                int64_t M, int64_t N, int64_t K,
                                const uint16_t *A, int64_t lda,
                                const uint16_t *B, int64_t ldb,
                                const float *C, int64_t ldc,
                                float alpha, float beta,
                                mpgemm_config *out);

/* MPGEMM_ECONFIG also when the entry was compiled for FP16 inputs. */
int mpgemm_bf16f32_layout_with_config(int config_id, int layout_a, int layout_b,
                                      int64_t M, int64_t N, int64_t K,
                                      const uint16_t *A, int64_t lda,
                                      const uint16_t *B, int64_t ldb,
                                      float *C, int64_t ldc,
                                      float alpha, float beta,
                                      void *stream);

/*
 * Everything in one call: input format (MPGEMM_IN_F16 or MPGEMM_IN_BF16),
 * storage orders (as for mpgemm_f16f32_layout) and an optional per-column
 * bias, the position-dependent epilogue of "Tensor cores with WMMA",
 * section "The habit this API takes away" (a bias per column):
 *
 *     C[i][j] <- alpha * sum_k A[i][k] * B[k][j] + beta * C[i][j] + bias[j]
 *
 * bias: N floats in device memory, 4-byte aligned, read-only, caller-owned;
 * NULL means no bias (the other entry points are this call with NULL).  The
 * bias is added in FP32 after the alpha and beta terms, also when alpha == 0
 * or K == 0 (then C <- beta*C + bias[j], C not read when beta == 0).
 * MPGEMM_ETYPE for an unknown input format; other errors as mpgemm_f16f32.
 */
int mpgemm_gemm_ex(int in_type, int layout_a, int layout_b,
                   int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb,
                   float *C, int64_t ldc,
                   float alpha, float beta,
                   const float *bias,
                   void *stream);

/* mpgemm_gemm_ex forced onto table entry `config_id` (tests and sweeps). */
int mpgemm_gemm_ex_with_config(int config_id, int in_type, int layout_a, int layout_b,
                               int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb,
                               float *C, int64_t ldc,
                               float alpha, float beta,
                               const float *bias,
                               void *stream);

/*
 * Split-K for products whose tile grid leaves compute units idle (few
 * output tiles, long K: the "skinny" 4096 x 16 x 4096 case of "Capstone 4: a
 * tensor-core GEMM", section "Independent gate").  The K range is cut into
 * `splits` pieces; each piece's workgroups write their unscaled FP32 partial
 * product to a caller-provided workspace, and a second kernel sums the
 * pieces in a fixed order (so results are run-to-run identical) and applies
 * alpha, beta and the bias:
 *
 *     C[i][j] <- alpha * sum_s P_s[i][j] + beta * C[i][j] + bias[j]
 *
 * mpgemm_splitk_plan reports, without any HIP call, how many pieces a call
 * would use (`splits_requested` 0: automatic, split only when K >= 4096
 * and the grid is under one wave of the workgroups the compute units hold
 * at once, into pieces of about 1024 K (at least 8 pieces for a grid of
 * at most 64 tiles, at least 6 for a larger one while it stays within 4
 * workgroups per compute unit), at most about 4 workgroups per compute
 * unit and at most 32 pieces; a product the factory gives the
 * narrow kernel stays whole when it
 * has at least 64 groups of 16 rows; n > 0: a tile kernel's K tiles dealt
 * into n pieces, at most one per K tile.  Every piece but the last holds
 * ceil(K tiles / pieces asked) K tiles, so the count can come out below the
 * one asked for, e.g. 2 pieces of 2 tiles for 3 asked of 4 tiles), the
 * workspace bytes that needs (splits*M*N*4; 0 when splits == 1) and the
 * kernel's table entry.  Output pointers may be
 * NULL.  Arguments as for mpgemm_gemm_ex; C, alpha and beta are not needed
 * to plan.
 *
 * mpgemm_gemm_splitk runs it: workspace is device memory the caller owns,
 * 4-byte aligned, at least the planned size (else MPGEMM_EWORKSPACE; NULL
 * with a non-zero plan is MPGEMM_ENULL); it may be NULL when the plan is a
 * single piece, which runs the ordinary path.  Calls that share a workspace
 * must not overlap in time.
 */
int mpgemm_splitk_plan(int in_type, int layout_a, int layout_b,
                       int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb,
                       int splits_requested,
                       int32_t *splits, int64_t *workspace_bytes, int32_t *config_id);

int mpgemm_gemm_splitk(int in_type, int layout_a, int layout_b,
                       int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb,
                       float *C, int64_t ldc,
                       float alpha, float beta,
                       const float *bias,
                       int splits_requested,
                       float *workspace, int64_t workspace_bytes,
                       void *stream);

/*
 * Split-K that allocates nothing, for callers that cannot call hipMalloc
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): mpgemm_gemm_splitk with the partial products in a static
 * array of MPGEMM_STATIC_SCRATCH_BYTES bytes that the library's code object
 * holds on each device it is loaded on, until the process ends, instead of
 * a caller workspace.  The plan is the one mpgemm_splitk_plan reports,
 * except that an automatic plan (`splits_requested` 0) whose workspace
 * exceeds the scratch takes as many pieces as fit (the unsplit product
 * when fewer than two do); a plan of one piece runs the ordinary path and
 * touches no scratch.  A requested plan whose workspace exceeds
 * MPGEMM_STATIC_SCRATCH_BYTES returns MPGEMM_ESCRATCH before any HIP call;
 * other errors as mpgemm_gemm_splitk.
 * The scratch is the current device's, so `stream` must belong to the
 * current device.  Every call on a device shares that device's scratch and
 * leaves its partial products there (each call writes every partial it then
 * reads, so nothing needs clearing): calls on one device whose kernels can
 * overlap in time (different streams without ordering between them) race
 * on it and give wrong results.  Thread-safe otherwise; the first call on a
 * device looks up the scratch's address there.
 */
#define MPGEMM_STATIC_SCRATCH_BYTES (32 * 1024 * 1024)

int mpgemm_gemm_splitk_static(int in_type, int layout_a, int layout_b,
                              int64_t M, int64_t N, int64_t K,
                              const uint16_t *A, int64_t lda,
                              const uint16_t *B, int64_t ldb,
                              float *C, int64_t ldc,
                              float alpha, float beta,
                              const float *bias,
                              int splits_requested,
                              void *stream);

/* Number of entries in the config table. */
int mpgemm_num_configs(void);

/* Table entry `config_id` into *out (grid = 0).  MPGEMM_ECONFIG if unknown. */
int mpgemm_config_info(int config_id, mpgemm_config *out);

/* Static text for an error code (never NULL). */
const char *mpgemm_strerror(int code);

/* Library version string, e.g. "mpgemm 0.8.0 gfx950". */
const char *mpgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MPGEMM_H */
