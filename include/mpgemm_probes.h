/*
 * mpgemm_probes.h -- diagnostics for the gfx950 GEMM library (AMD Instinct
 * MI355X), in a library of their own (libmpgemm_probes.so) so the product
 * library exports only the GEMM.
 *
 * They measure the properties the GEMM's design rests on: where a matrix
 * instruction puts each result (the lane layout the epilogue addresses), the
 * throughput the matrix cores sustain under the board's power limit, and the
 * rate at which the per-XCD L2 caches fill from the memory-side cache.  The
 * counterpart on the pages is the layout probe of "Tensor cores with WMMA"
 * (section "A warp owns a tile, and no thread owns an element": each lane
 * writes a marker into its accumulator slots and the owner map is printed)
 * and the profiler counters "Capstone 4: a tensor-core GEMM" reads (section
 * "Results").
 *
 * Every entry point takes device pointers the caller owns, enqueues one
 * kernel on `stream` (a hipStream_t passed as void*; NULL is the default
 * stream) and returns 0 (MPGEMM_OK) or a negative MPGEMM_E* code from
 * mpgemm.h; argument errors are found before any HIP call.  Nothing is
 * allocated and nothing synchronizes.
 */
#ifndef MPGEMM_PROBES_H
#define MPGEMM_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Runs one matrix-core instruction on known operands and writes where each
 * output element landed.  shape 32 uses the 32x32x16 FP16 instruction,
 * shape 16 the 16x16x32 one.  Operands: A[i][0] = i, A[i][1] = 1,
 * B[0][j] = 1, B[1][j] = S*j (S = 32 or 16), every other entry 0, so
 * D[i][j] = i + S*j exactly.  `out` is device memory for 64*16 floats
 * (shape 32) or 64*4 floats (shape 16): out[lane*V + v] = lane's v-th
 * accumulator.  MPGEMM_ECONFIG for another shape, MPGEMM_ENULL for NULL.
 */
int mpgemm_probe_mfma_layout(int shape, float *out, void *stream);

/*
 * Sustained matrix-core throughput with no memory traffic, for measuring
 * the clock and power the matrix cores settle at under load for given
 * operand values (the GEMM's inner loop is this instruction stream plus its
 * operand traffic).  `workgroups` workgroups of 8 waves; every wave loads
 * four operand pairs from `ops` once (ops_len >= 4096 16-bit values: pair
 * q, lane l reads 8 A values at (64*q + l)*16 and 8 B values right after)
 * and issues `iters` rounds of independent matrix instructions (8 of
 * 32x32x16 for shape 32, 32 of 16x16x32 for shape 16, i.e. 128 accumulator
 * registers per lane), rotating through the pairs.  FLOP per call =
 * workgroups * 8 waves * iters * 2*32*32*16 * 8 (shape 32) or
 * * 2*16*16*32 * 32 (shape 16).  Each thread writes the sum of its
 * accumulators to out[thread id] (out_len >= workgroups*512 floats).
 * in_type MPGEMM_IN_F16 or MPGEMM_IN_BF16.  MPGEMM_ECONFIG for another
 * format or shape, MPGEMM_ENULL for NULL buffers, MPGEMM_EDIM for short
 * buffers, iters outside 0..2^24 or workgroups outside 1..65535.
 */
int mpgemm_probe_mfma_rate(int in_type, int shape, const uint16_t *ops, int64_t ops_len, int64_t iters,
                           int workgroups, float *out, int64_t out_len, void *stream);

/* Request forms of mpgemm_probe_fill. */
#define MPGEMM_FILL_LDS16 0   /* buffer_load_dwordx4 ... lds: 16 B per lane into
                                 LDS (the GEMM's copy form), 1 KiB per wave
                                 instruction                                   */
#define MPGEMM_FILL_REG16 1   /* 16-byte buffer loads into registers           */
#define MPGEMM_FILL_REG4 2    /* 4-byte buffer loads into registers, 256 B per
                                 wave instruction                              */

/*
 * L2 fill rate per XCD.  `workgroups` (a multiple of 8, at most 65535)
 * workgroups of 8 waves; consecutive workgroup ids go round-robin to the 8
 * XCDs, so workgroup b runs on XCD b % 8.  XCD x reads a region of
 * `footprint` bytes: buf + x*footprint (shared == 0: each XCD its own data)
 * or buf (shared != 0: every XCD the same data, as the GEMM's panels are
 * read by several XCDs).  The XCD's workgroups form `replicas` groups
 * (replicas divides workgroups/8); each group sweeps the whole region once
 * per pass, its waves taking interleaved request-sized blocks (so with
 * replicas == 1 every byte is requested once per pass per XCD, and with
 * replicas == r by r compute units at about the same time, as the GEMM's
 * workgroups sharing a panel do).  `passes` sweeps.  Each wave keeps
 * `depth` (1, 2, 4, 8 or 16) requests in flight.  A region larger than the
 * 4 MiB L2 misses on every pass, so the time measures the fill from the
 * memory-side cache (which holds the whole buffer when it fits); a region
 * of 2 MiB or less stays in L2 and measures L2 hits.  Bytes per XCD per
 * call = footprint * passes * replicas (requested) and footprint * passes
 * (unique).  Register forms write each thread's XOR of what it loaded to
 * sink[thread id] (sink_len >= workgroups*512 floats; the LDS form writes
 * zeros there), so no load is dead.  `clocks` is NULL or device memory for
 * clocks_len >= 4 * workgroups uint64 values: workgroup b writes its shader
 * clock (s_memtime) at its start and end to clocks[4b], clocks[4b + 1] and
 * the constant 100 MHz clock (s_memrealtime) at its start and end to
 * clocks[4b + 2], clocks[4b + 3], so a caller can state a rate in bytes per
 * shader clock.
 * footprint: a positive multiple of 64 KiB with footprint * (shared ? 1 : 8)
 * <= buf_bytes < 2^31.  MPGEMM_ECONFIG for an unknown mode or depth,
 * MPGEMM_EDIM for any other size out of range, MPGEMM_ENULL for NULL buf or
 * sink, MPGEMM_EALIGN for a buffer that is not 16-byte aligned.
 */
int mpgemm_probe_fill(int mode, int depth, const void *buf, int64_t buf_bytes, int64_t footprint,
                      int shared, int replicas, int64_t passes, int workgroups, float *sink,
                      int64_t sink_len, uint64_t *clocks, int64_t clocks_len, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MPGEMM_PROBES_H */
