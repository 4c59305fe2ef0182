/*
 * oracle.c -- CPU oracle for the FP16-input, FP32-accumulate matrix product
 *
 *     C[i][j] <- alpha * sum_k A[i][k] * B[k][j] + beta * C[i][j]
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links it, and it shares no code, header, table or helper with the GPU path.
 *
 * What it follows (the method is the plain matrix product, so the oracle is
 * that definition written out):
 *   - "Capstone 4: a tensor-core GEMM", Minimal model: A and B are stored as
 *     FP16, the sum and C are wider (FP32 on the GPU).  Here every input is
 *     widened exactly to FP64 and the sum is carried in FP64, which is the
 *     "double-precision CPU result" the same page checks every element against
 *     (section "Compare like with like").
 *   - Row-major A (M x K, leading dimension lda), row-major B (K x N, ldb),
 *     row-major C (M x N, ldc), all leading dimensions counted in elements.
 *     The *_layout entry points also take A and/or B stored column-major
 *     (A[i][k] at A[k*lda + i], B[k][j] at B[j*ldb + k]), the layout of the
 *     same page's "Independent gate" (A row-major, B column-major); only the
 *     element addressing changes, the arithmetic is the same.
 *   - beta == 0 means C is not read at all (the output may hold NaN poison,
 *     "02_mixed_precision_gemm", Verification).
 *
 * BF16 inputs (the other 16-bit tensor-core input type "Tensor cores with
 * WMMA" lists, section "A warp owns a tile, and no thread owns an element")
 * go through the *_bf16_* entry points: the same product, with each input
 * decoded from the bfloat16 format instead (8 significant bits; products of
 * two are exact in FP64 just the same, and every finite BF16 value and
 * product is in FP64's range).
 *
 * A per-column bias (the position-dependent epilogue "Tensor cores with WMMA"
 * names in section "The habit this API takes away": a bias per column, which
 * a WMMA fragment cannot place but a documented accumulator layout can) is
 * taken by the *_ex entry points: ref[i][j] = alpha*s + beta*c + bias[j],
 * each term in FP64.
 *
 * Arithmetic: an FP16 value is an integer times 2^-24 with at most 11
 * significant bits, so its FP64 widening is exact and every product of two
 * widened values is exact in FP64 (22 significant bits).  Only the running
 * sum rounds, in ascending k order, with error at most K * 2^-53 * sum|a*b|.
 * Build with -O2 -fno-fast-math -ffp-contract=off so the compiler neither
 * reassociates the sum nor fuses alpha*s + beta*c.
 *
 * Parallelism: rows are split across OpenMP threads; each output element is
 * computed by one thread in the same order, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      : zero or subnormal, value = fraction * 2^-24
 *   exponent 1..30  : normal, value = (1024 + fraction) * 2^(exponent - 25)
 *   exponent 31     : infinity (fraction 0) or NaN (fraction != 0)
 */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int exponent = (h >> 10) & 0x1f;
    const int fraction = h & 0x3ff;
    double v;
    if (exponent == 0) {
        v = ldexp((double)fraction, -24);
    } else if (exponent == 31) {
        v = (fraction == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + fraction), exponent - 25);
    }
    return sign ? -v : v;
}

void oracle_f16_to_f64_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f64(h[i]);
}

/*
 * bfloat16 -> binary64, from the format's definition: the upper half of an
 * IEEE binary32, i.e. 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 *   exponent 0      : zero or subnormal, value = fraction * 2^-133
 *   exponent 1..254 : normal, value = (128 + fraction) * 2^(exponent - 134)
 *   exponent 255    : infinity (fraction 0) or NaN (fraction != 0)
 */
double oracle_bf16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int exponent = (h >> 7) & 0xff;
    const int fraction = h & 0x7f;
    double v;
    if (exponent == 0) {
        v = ldexp((double)fraction, -133);
    } else if (exponent == 255) {
        v = (fraction == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(128 + fraction), exponent - 134);
    }
    return sign ? -v : v;
}

void oracle_bf16_to_f64_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f64(h[i]);
}

/*
 * Element strides of the two operands: A[i][k] is A[i*a_i + k*a_k] and
 * B[k][j] is B[k*b_k + j*b_j].
 */
typedef struct {
    int64_t a_i, a_k, b_k, b_j;
    double (*decode)(uint16_t);  /* FP16 or BF16 bits -> FP64 */
    const float *bias;           /* per-column bias (N values) or NULL */
} strides_t;

#define ORACLE_ROW_MAJOR 0
#define ORACLE_COL_MAJOR 1

static strides_t strides_for(int layout_a, int layout_b, int64_t lda, int64_t ldb)
{
    strides_t t;
    t.a_i = layout_a == ORACLE_COL_MAJOR ? 1 : lda;
    t.a_k = layout_a == ORACLE_COL_MAJOR ? lda : 1;
    t.b_k = layout_b == ORACLE_COL_MAJOR ? 1 : ldb;
    t.b_j = layout_b == ORACLE_COL_MAJOR ? ldb : 1;
    t.decode = oracle_f16_to_f64;
    t.bias = NULL;
    return t;
}

/*
 * One output element: the dot product of row i of A with column j of B in
 * ascending k, then alpha*s + beta*c.  Also returns sum_k |a_ik * b_kj|, the
 * scale the acceptance rule is written against.
 *
 * When alpha == 0 or K == 0 the product term is not formed at all and A and
 * B are not read: the result is beta*c (+ bias), and the sum of |a*b| is 0.
 * The pages say nothing about this case; the reading taken is the usual
 * convention of matrix-product interfaces (the counterpart of "beta == 0
 * means C is not read"), so a NaN or Inf in A or B, or a non-finite alpha
 * with K == 0, does not reach the result.
 */
static void entry(int64_t i, int64_t j, int64_t K,
                  const uint16_t *A, const uint16_t *B, strides_t st,
                  const float *C, int64_t ldc,
                  double alpha, double beta,
                  double *ref, double *absdot)
{
    const int product = alpha != 0.0 && K > 0;
    double s = 0.0;
    double s_abs = 0.0;
    for (int64_t k = 0; product && k < K; ++k) {
        const double a = st.decode(A[i * st.a_i + k * st.a_k]);
        const double b = st.decode(B[k * st.b_k + j * st.b_j]);
        const double p = a * b; /* exact */
        s += p;
        s_abs += fabs(p);
    }
    double r;
    if (product) {
        r = alpha * s;
        if (beta != 0.0)
            r += beta * (double)C[i * ldc + j];
    } else {
        r = beta != 0.0 ? beta * (double)C[i * ldc + j] : 0.0;
    }
    if (st.bias)
        r += (double)st.bias[j];
    *ref = r;
    if (absdot)
        *absdot = s_abs;
}

/* Error codes shared by both entry points. */
#define ORACLE_OK 0
#define ORACLE_EBADDIM (-1)
#define ORACLE_EBADLD (-2)
#define ORACLE_ENULL (-3)
#define ORACLE_EBADLAYOUT (-4)

/* A stored row-major needs lda >= K, column-major lda >= M; B row-major
 * needs ldb >= N, column-major ldb >= K; C (always row-major) ldc >= N. */
static int check_args(int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                      const uint16_t *A, int64_t lda,
                      const uint16_t *B, int64_t ldb,
                      const float *C, int64_t ldc, double beta)
{
    if ((layout_a != ORACLE_ROW_MAJOR && layout_a != ORACLE_COL_MAJOR) ||
        (layout_b != ORACLE_ROW_MAJOR && layout_b != ORACLE_COL_MAJOR))
        return ORACLE_EBADLAYOUT;
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_EBADDIM;
    const int64_t a_row = layout_a == ORACLE_COL_MAJOR ? M : K;
    const int64_t b_row = layout_b == ORACLE_COL_MAJOR ? K : N;
    if (lda < (a_row > 1 ? a_row : 1) || ldb < (b_row > 1 ? b_row : 1) || ldc < (N > 1 ? N : 1))
        return ORACLE_EBADLD;
    if (M > 0 && N > 0 && K > 0 && (A == NULL || B == NULL))
        return ORACLE_ENULL;
    if (M > 0 && N > 0 && beta != 0.0 && C == NULL)
        return ORACLE_ENULL;
    return ORACLE_OK;
}

/*
 * Full product with the given storage orders of A and B.  ref and absdot
 * (absdot may be NULL) are M x N, row-major, packed (leading dimension N),
 * owned by the caller.
 */
static int gemm_full(int bf16, int layout_a, int layout_b,
                     int64_t M, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda,
                     const uint16_t *B, int64_t ldb,
                     const float *C, int64_t ldc,
                     double alpha, double beta, const float *bias,
                     double *ref, double *absdot)
{
    const int rc = check_args(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, beta);
    if (rc != ORACLE_OK)
        return rc;
    if (M > 0 && N > 0 && ref == NULL)
        return ORACLE_ENULL;
    strides_t st = strides_for(layout_a, layout_b, lda, ldb);
    if (bf16)
        st.decode = oracle_bf16_to_f64;
    st.bias = bias;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            entry(i, j, K, A, B, st, C, ldc, alpha, beta,
                  &ref[i * N + j], absdot ? &absdot[i * N + j] : NULL);
        }
    }
    return ORACLE_OK;
}

int oracle_gemm_layout(int layout_a, int layout_b,
                       int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb,
                       const float *C, int64_t ldc,
                       double alpha, double beta,
                       double *ref, double *absdot)
{
    return gemm_full(0, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, NULL,
                     ref, absdot);
}

/* The same product with BF16 inputs. */
int oracle_gemm_bf16_layout(int layout_a, int layout_b,
                            int64_t M, int64_t N, int64_t K,
                            const uint16_t *A, int64_t lda,
                            const uint16_t *B, int64_t ldb,
                            const float *C, int64_t ldc,
                            double alpha, double beta,
                            double *ref, double *absdot)
{
    return gemm_full(1, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, NULL,
                     ref, absdot);
}

/* Full product, A and B row-major. */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb,
                const float *C, int64_t ldc,
                double alpha, double beta,
                double *ref, double *absdot)
{
    return oracle_gemm_layout(ORACLE_ROW_MAJOR, ORACLE_ROW_MAJOR, M, N, K, A, lda, B, ldb,
                              C, ldc, alpha, beta, ref, absdot);
}

/*
 * Selected entries only: element t of the output is (rows[t], cols[t]).
 * Used where the full product would take too long on the CPU.
 */
static int gemm_entries(int bf16, int layout_a, int layout_b,
                        int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb,
                        const float *C, int64_t ldc,
                        double alpha, double beta, const float *bias,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        double *ref, double *absdot)
{
    const int rc = check_args(layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, beta);
    if (rc != ORACLE_OK)
        return rc;
    if (count < 0)
        return ORACLE_EBADDIM;
    for (int64_t t = 0; t < count; ++t) {
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_EBADDIM;
    }
    strides_t st = strides_for(layout_a, layout_b, lda, ldb);
    if (bf16)
        st.decode = oracle_bf16_to_f64;
    st.bias = bias;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        entry(rows[t], cols[t], K, A, B, st, C, ldc, alpha, beta,
              &ref[t], absdot ? &absdot[t] : NULL);
    }
    return ORACLE_OK;
}

int oracle_gemm_layout_entries(int layout_a, int layout_b,
                               int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb,
                               const float *C, int64_t ldc,
                               double alpha, double beta,
                               int64_t count, const int64_t *rows, const int64_t *cols,
                               double *ref, double *absdot)
{
    return gemm_entries(0, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, NULL,
                        count, rows, cols, ref, absdot);
}

int oracle_gemm_bf16_layout_entries(int layout_a, int layout_b,
                                    int64_t M, int64_t N, int64_t K,
                                    const uint16_t *A, int64_t lda,
                                    const uint16_t *B, int64_t ldb,
                                    const float *C, int64_t ldc,
                                    double alpha, double beta,
                                    int64_t count, const int64_t *rows, const int64_t *cols,
                                    double *ref, double *absdot)
{
    return gemm_entries(1, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, NULL,
                        count, rows, cols, ref, absdot);
}

/* Selected entries, A and B row-major. */
int oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb,
                        const float *C, int64_t ldc,
                        double alpha, double beta,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        double *ref, double *absdot)
{
    return oracle_gemm_layout_entries(ORACLE_ROW_MAJOR, ORACLE_ROW_MAJOR, M, N, K, A, lda, B, ldb,
                                      C, ldc, alpha, beta, count, rows, cols, ref, absdot);
}

/*
 * Everything at once: input format (bf16 = 0: FP16, 1: BF16), storage
 * orders, and an optional per-column bias (NULL for none).
 */
int oracle_gemm_ex(int bf16, int layout_a, int layout_b,
                   int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb,
                   const float *C, int64_t ldc,
                   double alpha, double beta, const float *bias,
                   double *ref, double *absdot)
{
    return gemm_full(bf16 != 0, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                     bias, ref, absdot);
}

int oracle_gemm_ex_entries(int bf16, int layout_a, int layout_b,
                           int64_t M, int64_t N, int64_t K,
                           const uint16_t *A, int64_t lda,
                           const uint16_t *B, int64_t ldb,
                           const float *C, int64_t ldc,
                           double alpha, double beta, const float *bias,
                           int64_t count, const int64_t *rows, const int64_t *cols,
                           double *ref, double *absdot)
{
    return gemm_entries(bf16 != 0, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                        bias, count, rows, cols, ref, absdot);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
