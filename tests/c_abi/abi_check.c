/*
 * abi_check.c -- the GEMM called from plain C, with no Python and no torch:
 * device buffers come from the HIP runtime, and the library is called
 * through mpgemm.h only.
 *
 * A and B hold small integers (A in [-3,3], B in [-2,2]: the exact-integer
 * fill of "Tensor cores with WMMA", section "Why this program calls cuBLAS
 * twice"), so every partial sum is an integer below 2^24 and the FP32 result
 * must equal the integer product exactly.  The shape fits no tile, every
 * leading dimension is padded, C starts as NaN (beta = 0 must not read it)
 * and the padding columns of C must stay untouched.  A second call with
 * alpha = 2, beta = -1 turns C into 2*A*B - A*B = A*B, exactly.  Argument
 * errors must come back before any launch.
 *
 * Exit status 0 and one "ok" line on success; 1 and a message otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mpgemm.h"

/* FP16 bit pattern of a small integer (-3..3): sign bit, and 1.0 = 0x3C00,
 * 2.0 = 0x4000, 3.0 = 0x4200 (binary16: exponent bias 15, 10 fraction bits). */
static uint16_t f16_small_int(int v)
{
    static const uint16_t mag[4] = {0x0000, 0x3C00, 0x4000, 0x4200};
    return (uint16_t)((v < 0 ? 0x8000 : 0) | mag[v < 0 ? -v : v]);
}

static uint32_t lcg(uint32_t *s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

#define CHECK_HIP(x)                                                      \
    do {                                                                  \
        hipError_t e_ = (x);                                              \
        if (e_ != hipSuccess) {                                           \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));       \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main(void)
{
    const int64_t M = 333, N = 257, K = 617;
    const int64_t lda = K + 3, ldb = N + 5, ldc = N + 2;
    int *ai = malloc(sizeof(int) * M * K), *bi = malloc(sizeof(int) * K * N);
    uint16_t *ha = malloc(2 * M * lda), *hb = malloc(2 * K * ldb);
    float *hc = malloc(4 * M * ldc);
    if (!ai || !bi || !ha || !hb || !hc)
        return 1;
    uint32_t seed = 12345u;
    memset(ha, 0xFF, 2 * M * lda); /* NaN in the padding */
    memset(hb, 0xFF, 2 * K * ldb);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) {
            ai[i * K + k] = (int)(lcg(&seed) % 7) - 3;
            ha[i * lda + k] = f16_small_int(ai[i * K + k]);
        }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            bi[k * N + j] = (int)(lcg(&seed) % 5) - 2;
            hb[k * ldb + j] = f16_small_int(bi[k * N + j]);
        }
    memset(hc, 0xFF, 4 * M * ldc); /* NaN everywhere, padding included */

    uint16_t *da, *db;
    float *dc;
    CHECK_HIP(hipMalloc((void **)&da, 2 * M * lda));
    CHECK_HIP(hipMalloc((void **)&db, 2 * K * ldb));
    CHECK_HIP(hipMalloc((void **)&dc, 4 * M * ldc));
    CHECK_HIP(hipMemcpy(da, ha, 2 * M * lda, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(db, hb, 2 * K * ldb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dc, hc, 4 * M * ldc, hipMemcpyHostToDevice));

    if (mpgemm_f16f32(-1, N, K, da, lda, db, ldb, dc, ldc, 1.0f, 0.0f, NULL) != MPGEMM_EDIM ||
        mpgemm_f16f32(M, N, K, da, K - 1, db, ldb, dc, ldc, 1.0f, 0.0f, NULL) != MPGEMM_ELD ||
        mpgemm_f16f32(M, N, K, NULL, lda, db, ldb, dc, ldc, 1.0f, 0.0f, NULL) != MPGEMM_ENULL) {
        fprintf(stderr, "argument errors not reported\n");
        return 1;
    }
    for (int pass = 0; pass < 2; ++pass) {
        const float alpha = pass == 0 ? 1.0f : 2.0f, beta = pass == 0 ? 0.0f : -1.0f;
        const int rc = mpgemm_f16f32(M, N, K, da, lda, db, ldb, dc, ldc, alpha, beta, NULL);
        if (rc != MPGEMM_OK) {
            fprintf(stderr, "mpgemm_f16f32: %s\n", mpgemm_strerror(rc));
            return 1;
        }
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(hc, dc, 4 * M * ldc, hipMemcpyDeviceToHost));
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) {
                long s = 0;
                for (int64_t k = 0; k < K; ++k)
                    s += (long)ai[i * K + k] * bi[k * N + j];
                if (hc[i * ldc + j] != (float)s) {
                    fprintf(stderr, "pass %d: C[%lld][%lld] = %.9g, want %ld\n", pass, (long long)i,
                            (long long)j, hc[i * ldc + j], s);
                    return 1;
                }
            }
            for (int64_t j = N; j < ldc; ++j)
                if (!isnan(hc[i * ldc + j])) {
                    fprintf(stderr, "padding column %lld of row %lld was written\n", (long long)j,
                            (long long)i);
                    return 1;
                }
        }
    }
    CHECK_HIP(hipFree(da));
    CHECK_HIP(hipFree(db));
    CHECK_HIP(hipFree(dc));
    printf("abi_check %lldx%lldx%lld (%s): ok\n", (long long)M, (long long)N, (long long)K, mpgemm_version());
    free(ai);
    free(bi);
    free(ha);
    free(hb);
    free(hc);
    return 0;
}
