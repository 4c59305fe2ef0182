// kernels.hpp -- gfx950 device code for C = alpha*A*B + beta*C with FP16 A, B
// and FP32 accumulation and output (the mixed-precision contract of
// "Capstone 4: a tensor-core GEMM", sections "Capability" and "Minimal model").
//
// Kernels:
//   gemm_pipe<Cfg>    block tile staged through an LDS ring of K tiles filled by
//                     direct-to-LDS buffer loads, wave tiles on
//                     v_mfma_f32_32x32x16_f16 or v_mfma_f32_16x16x32_f16,
//                     bounds-checked alpha/beta (+ bias) epilogue.  The pages'
//                     staged-tile design ("Capstone 4", Worked path, and the
//                     double-buffered copy of "02_mixed_precision_gemm",
//                     Summary) is the prior art; the layout below is gfx950's.
//   gemm_narrow       N <= 16: 16 rows of C per workgroup, K split over waves.
//   gemm_direct       one 32x32 MFMA tile per wave with operands loaded
//                     straight from memory, 64-bit addressing, any size,
//                     stride and storage order: the universal fallback.
//   splitk_reduce     sums split-K partial products in a fixed order.
//   scale_c           C <- beta*C when alpha == 0 or K == 0.
//
// Matrix-core lane layouts used here (CDNA3/CDNA4 matrix instruction docs,
// checked on the device by the layout probe of the diagnostics library):
//   v_mfma_f32_32x32x16_f16: lane l supplies A[l%32][8*(l/32) + 0..7] and
//     B[8*(l/32) + 0..7][l%32]; accumulator v (0..15) of lane l holds
//     D[8*(v/4) + 4*(l/32) + v%4][l%32].
//   v_mfma_f32_16x16x32_f16: lane l supplies A[l%16][8*(l/16) + 0..7] and
//     B[8*(l/16) + 0..7][l%16]; accumulator v (0..3) holds D[4*(l/16) + v][l%16].
// Any permutation of k that A and B share gives the same sum, so only the
// row/column placement matters for correctness.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace mpg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource: raw (stride 0) byte-addressed buffer.  Word 3 is the
// gfx9-family data-format word.  A load whose byte offset is >= num_records
// returns zero; the kernels send every out-of-range element to kOOB, which
// is how ragged M, N and K edges read zeros without host padding.
constexpr int32_t kNumRecords = 0x7FFFFFFF;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int32_t kRsrcWord3 = 0x00020000;

// Cache-policy bits of a buffer store: non-temporal (streaming) write.
constexpr int32_t kStoreNT = 2;

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// each with a private L2.
constexpr int kNumXcd = 8;

#ifdef MPGEMM_TIMELINE
// Timeline build only (libmpgemm_timeline.so, a diagnostics library; the
// product library compiles none of this).  The pipelined kernel records, for
// each of the first kTimelineWgs workgroups of a launch, when it started,
// when each of its first kTimelineTiles K tiles was published, and when its
// K loop and its epilogue ended (slot layout in mpgemm_timeline.h).  Thread 0
// keeps the stamps in LDS while the kernel runs -- LDS writes do not count
// against the vector memory counter the ring's waits rely on -- and copies
// them to g_timeline after its last store.
constexpr int kTimelineSlots = 48;
constexpr int kTimelineWgs = 4096;
constexpr int kTimelineTiles = 41;
__device__ uint64_t g_timeline[kTimelineWgs * kTimelineSlots];
#endif

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             kNumRecords, kRsrcWord3);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi)
{
    return (lo & 0xFFFFu) | (hi << 16);
}

// Same, but only the first `nvalid` (1..7) elements are in range; the rest
// read as zero.  Used where a vector straddles the end of a row.
__device__ __forceinline__ u32x4 load8_partial(__amdgpu_buffer_rsrc_t r, uint32_t off, int nvalid)
{
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        h[e] = __builtin_amdgcn_raw_buffer_load_b16(r, e < nvalid ? off + 2u * e : kOOB, 0, 0);
    return u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
}

struct GemmArgs {
    const uint16_t *A;
    const uint16_t *B;
    float *C;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    // element strides: A[i][k] at A[i*a_i + k*a_k], B[k][j] at B[k*b_k + j*b_j]
    // (read by the direct kernel; the tiled kernels compile their layout in)
    int64_t a_i, a_k, b_k, b_j;
    float alpha, beta;
    // optional per-column bias: C[i][j] gains bias[j] (nullptr: none)
    const float *bias;
    int32_t tiles_m, tiles_n;
    int32_t group_m;
    // split-K (pipelined kernel only): when splits > 1 the grid holds
    // `splits` copies of the tile grid; copy s sums k in [s*k_split,
    // (s+1)*k_split) and writes its unscaled partial tile to ws + s*M*N (rows
    // of N), which a reduction then combines in a fixed order.
    int32_t splits;
    int64_t k_split;
    float *ws;
};

// Input format of A and B: IEEE binary16 or bfloat16.  Both are 16-bit
// patterns to every copy and LDS read; only the matrix instruction differs.
constexpr int kInF16 = 0;
constexpr int kInBF16 = 1;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// acc += A_op * B_op on the 32x32x16 matrix instruction of the input format.
template <int IN>
__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 acc)
{
    if constexpr (IN == kInBF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}

// acc += A_op * B_op on the 16x16x32 matrix instruction of the input format.
template <int IN>
__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 acc)
{
    if constexpr (IN == kInBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// Workgroup id -> (tile row, tile column).  First undo the round-robin XCD
// dispatch so each XCD owns one contiguous run of tile ids, then walk that
// run in groups of `group_m` tile rows so the workgroups resident on one XCD
// at the same time share A row-panels and B column-panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int nb, int tiles_n, int tiles_m, int group_m,
                                            int &tm, int &tn)
{
    const int xcd = bid % kNumXcd;
    const int local = bid / kNumXcd;
    const int per = nb / kNumXcd;
    const int rem = nb % kNumXcd;
    const int t = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    const int group = group_m * tiles_n;
    const int first_m = (t / group) * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int in_group = t % group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Bounds-checked epilogue for one 32x32 accumulator tile whose top-left
// element is C[row0][col0]: C = alpha*acc + beta*C, C not read when beta == 0.
__device__ __forceinline__ void store_tile32(const floatx16 &acc, float *C, int64_t ldc,
                                             int64_t M, int64_t N, int64_t row0, int64_t col0,
                                             float alpha, float beta, const float *bias, int lane)
{
    const int64_t col = col0 + (lane & 31);
    if (col >= N)
        return;
    const float bv = bias ? bias[col] : 0.0f;
    const int64_t rbase = row0 + 4 * (lane >> 5);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t row = rbase + 8 * (v >> 2) + (v & 3);
        if (row < M) {
            float *p = C + row * ldc + col;
            const float s = acc[v];
            float val = (beta == 0.0f) ? alpha * s : __builtin_fmaf(alpha, s, beta * *p);
            if (bias)
                val += bv;
            *p = val;
        }
    }
}

// ---------------------------------------------------------------------------
// Direct kernel: 4 waves, 64x64 of C per workgroup, operands from memory.
// ---------------------------------------------------------------------------
template <int IN>
__global__ void __launch_bounds__(256)
gemm_direct(GemmArgs args)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tm = blockIdx.x / args.tiles_n;
    const int64_t tn = blockIdx.x % args.tiles_n;
    const int64_t row0 = tm * 64 + (wave >> 1) * 32;
    const int64_t col0 = tn * 64 + (wave & 1) * 32;
    const int64_t ra = row0 + (lane & 31);
    const int64_t cb = col0 + (lane & 31);
    const bool ra_ok = ra < args.M;
    const bool cb_ok = cb < args.N;
    const int kbase = 8 * (lane >> 5);
    floatx16 acc = floatx16{0};
    for (int64_t k0 = 0; k0 < args.K; k0 += 16) {
        half8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + kbase + e;
            const bool k_ok = k < args.K;
            const uint16_t av = (ra_ok && k_ok) ? args.A[ra * args.a_i + k * args.a_k] : (uint16_t)0;
            const uint16_t bv = (cb_ok && k_ok) ? args.B[k * args.b_k + cb * args.b_j] : (uint16_t)0;
            a[e] = __builtin_bit_cast(_Float16, av);
            b[e] = __builtin_bit_cast(_Float16, bv);
        }
        acc = mfma32<IN>(a, b, acc);
    }
    store_tile32(acc, args.C, args.ldc, args.M, args.N, row0, col0, args.alpha, args.beta, args.bias,
                 lane);
}

// Split-K reduction: C <- alpha * sum_{s<splits} ws[s] + beta*C (+ bias[j]),
// the partials summed in ascending s (run-to-run deterministic).  ws holds
// `splits` row-major M x N partial products, rows of N.  Grid-stride over
// rows in y and columns in x.
__global__ void __launch_bounds__(256)
splitk_reduce(float *C, int64_t M, int64_t N, int64_t ldc, const float *ws, int splits,
              float alpha, float beta, const float *bias)
{
    for (int64_t i = blockIdx.y; i < M; i += gridDim.y) {
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < N;
             j += (int64_t)gridDim.x * blockDim.x) {
            float acc = 0.0f;
            for (int s = 0; s < splits; ++s)
                acc += ws[(int64_t)s * M * N + i * N + j];
            float *p = C + i * ldc + j;
            float v = alpha * acc;
            if (beta != 0.0f)
                v = __builtin_fmaf(beta, *p, v);
            if (bias)
                v += bias[j];
            *p = v;
        }
    }
}

// C <- beta*C (+ bias[j]); beta == 0 writes without reading C.  Grid-stride
// over rows in y and columns in x.
__global__ void __launch_bounds__(256)
scale_c(float *C, int64_t M, int64_t N, int64_t ldc, float beta, const float *bias)
{
    for (int64_t i = blockIdx.y; i < M; i += gridDim.y) {
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < N;
             j += (int64_t)gridDim.x * blockDim.x) {
            float *p = C + i * ldc + j;
            float v = (beta == 0.0f) ? 0.0f : beta * *p;
            if (bias)
                v += bias[j];
            *p = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel: global -> LDS with buffer_load ... lds
// ---------------------------------------------------------------------------
// Each operand tile of a stage sits in LDS in its storage order, in one of two
// forms (BK = 32, 64 or 128; BX = BM for A, BN for B):
//   K-contiguous: one LDS row of BK values (2*BK bytes) per M row of A
//     (row-major A) or per N column of B (column-major B).  Operands are read
//     with ds_read_b128: lane l takes the 8 K-consecutive values of row l%32
//     at logical chunk 2*ks + l/32 (32x32x16 instruction), or of row l%16 at
//     chunk 4*ks + l/16 (16x16x32).
//   outer-contiguous: one LDS row of BX values per k, as a row-major B or a
//     column-major A holds them in memory.  Operands are read with the
//     transposing ds_read_b64_tr_b16, two per operand.
// gfx950's LDS has 64 banks of 4 bytes: a ds_read_b128 serves 16 lanes per
// cycle and a ds_read_b64 (including the transposing read) 32 lanes, so each
// such group must touch 256 distinct bytes of bank space to run at full rate.
// The 16-byte chunk c of LDS row r sits at physical chunk c ^ swz(r):
//   K-contiguous: one 16-lane group reads 16 consecutive rows at one logical
//     chunk.  With 128-byte rows two rows share a 256-byte bank window, so
//     swz(r) = (r >> 1) & 7 gives the 8 rows of each parity 8 distinct chunks;
//     with 64-byte rows four rows share a window and swz(r) = (r >> 2) & 3; a
//     256-byte row fills the window by itself and swz(r) = r & 15.
//   outer-contiguous, 32x32x16 instruction: one 32-lane group of the
//     transposing read touches 4 consecutive rows x 4 consecutive chunks;
//     swz(k) = 4*(k & 3) moves the rows to 4 different 64-byte quarters of the
//     window (rows of 256 bytes or more), or 4*((k >> 1) & 1) for 128-byte
//     rows (BX = 64), where row parity already selects the window half.
//   outer-contiguous, 16x16x32 instruction: the group touches rows
//     {0,1,2,3} and {8,9,10,11} (plus a multiple of 4 that keeps these
//     bits) x 2 consecutive chunks, the first even; swz(k) = 2*(k & 3) +
//     8*((k >> 3) & 1) gives the 8 rows 8 distinct chunk pairs (rows of 256
//     bytes or more), and 2*((k >> 1) & 1) + 4*((k >> 3) & 1) does the same
//     within each half window for 128-byte rows.
// Copies: one wave instruction of buffer_load_dwordx4 ... lds writes 64
// lanes x 16 B to LDS at M0 + 16*lane (a contiguous KiB); the swizzle is
// applied by choosing which global chunk each lane fetches.  Lanes whose
// chunk is outside the matrix get an offset past num_records and write
// zeros.  Vectors that straddle the end of a row are filled through
// registers instead.  The 16-byte loads need only the operands' 2-byte
// alignment: under ROCm, gfx9-family devices run vector memory in unaligned
// mode (the kernel driver sets it for every process), where a 16-byte buffer
// load at any 2-byte aligned address returns exactly the bytes there, into
// registers and through the LDS-DMA form alike.  Without that mode the
// hardware would drop the low address bits and read the wrong bytes; the GPU
// tests on 2-byte aligned operands (offset pointers, odd leading
// dimensions) check it on every device they run on.
//
// Schedule (per wave, per K tile of BK): each k-step first issues every
// operand read of the next k-step (into the other register set), then runs
// its MFMAs in groups of FN.  The barrier that publishes tile t+1 sits
// before the last k-step of tile t, so the reads of tile t+1's first k-step
// overlap that k-step's MFMAs.  Past that barrier no wave reads tile t's
// buffer again, and the copies of tile t+STAGES into it start at once,
// spread over the following MFMA groups: the copy engine is never left
// without work while a buffer is free.
typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Storage order of an operand in memory (C is always row-major).
constexpr int kRowMajor = 0;
constexpr int kColMajor = 1;


// One operand tile in LDS.  KC = true: K-contiguous rows (BX rows of BK);
// KC = false: outer-contiguous rows (BK rows of BX).  NW waves share the
// copies; each copy instruction fills RPI whole LDS rows.
template <int BX, int BK, bool KC, int NW, int MI = 32>
struct OpTile {
    static constexpr bool K_CONTIG = KC;
    static constexpr int NWAVES = NW;
    static constexpr int ROWS = KC ? BX : BK;
    static constexpr int ROWB = 2 * (KC ? BK : BX);   // bytes per LDS row
    static constexpr int CH = ROWB / 16;               // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;                // rows per copy instruction
    static constexpr int PW = ROWS / RPI / NW;         // copies per wave per tile
    static constexpr int BYTES = ROWS * ROWB;
    static_assert(64 % CH == 0, "a row must hold at most 64 chunks");
    static_assert(KC ? (CH == 4 || CH == 8 || CH == 16) : CH >= 8,
                  "no conflict-free swizzle for this row width");
    static_assert((ROWS / RPI) % NW == 0, "copies must split evenly over waves");
    __device__ static __forceinline__ int swz(int r)
    {
        if constexpr (KC)
            return CH == 16 ? (r & 15) : CH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
        else if constexpr (MI == 32)
            return CH >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
        else
            return CH >= 16 ? 2 * (r & 3) + 8 * ((r >> 3) & 1) : 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1);
    }
};

// KGROUPS > 1 splits the waves of a workgroup into groups that share every
// LDS tile but take different k-steps of it, each group covering the whole
// BM x BN block with WAVES_M x WAVES_N waves; the groups' sums are added in
// LDS at the end.  For a small block this keeps the wave tiles large (fewer
// LDS bytes per matrix instruction) while two waves per SIMD still hide
// latency.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_,
          int LAYOUT_A_ = kRowMajor, int LAYOUT_B_ = kRowMajor, int IN_ = kInF16, int KGROUPS_ = 1,
          int MI_ = 32, int STAGGER_ = 0>
struct PipeCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int LAYOUT_A = LAYOUT_A_, LAYOUT_B = LAYOUT_B_;
    static constexpr int IN = IN_;
    static constexpr int KGROUPS = KGROUPS_;
    // K order.  0: every workgroup walks the K tiles from the first.  D >= 2:
    // the workgroup at tile row tm, tile column tn starts at K tile
    // (tm + tn) mod min(D, K tiles) and wraps around, so the workgroups of
    // an XCD that share an A or B panel request its lines at D different
    // times instead of all at once: one of them misses in the L2 and the
    // others, up to D - 1 K tiles later, hit.
    static constexpr int STAGGER = STAGGER_;
    // matrix instruction: 32 = 32x32x16 (16 accumulators per lane),
    // 16 = 16x16x32 (4 accumulators per lane)
    static constexpr int MI = MI_;
    static constexpr int KD = MI == 32 ? 16 : 32;         // K of one instruction
    static constexpr int AV = MI == 32 ? 16 : 4;          // accumulators per lane
    static constexpr int NWG = WAVES_M * WAVES_N;         // waves per k-group
    static constexpr int NW = NWG * KGROUPS;              // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / MI, FN = WTN / MI;
    static constexpr int KS = BK / KD;                    // MFMA k-steps per tile
    static constexpr int KSL = KS / KGROUPS;              // ... taken by each k-group
    // row-major A and column-major B are K-contiguous in memory
    using TA = OpTile<BM, BK, LAYOUT_A == kRowMajor, NW, MI>;
    using TB = OpTile<BN, BK, LAYOUT_B == kColMajor, NW, MI>;
    static constexpr int A_BYTES = TA::BYTES;
    static constexpr int B_BYTES = TB::BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int APW = TA::PW, BPW = TB::PW;      // copies per wave per tile
    static constexpr int NL = APW + BPW;                   // vmcnt per tile
    static constexpr int NCOPY = APW + BPW;                // copy instructions per wave per tile
    // MFMA groups (FM per k-step) over which a tile's copies are spread,
    // counted from the barrier that frees their buffer.  With two stages the
    // copies must land one tile later, so they go out one per group, at
    // about the rate the memory system serves them, leaving the rest of the
    // tile as slack; deeper rings spread them over a whole tile.
    static constexpr int COPY_WINDOW =
        STAGES == 2 ? (NCOPY < KSL * FM ? (NCOPY > 0 ? NCOPY : 1) : KSL * FM) : KSL * FM;
    static_assert(KGROUPS >= 1 && KS % KGROUPS == 0, "k-steps must split evenly over k-groups");
    static_assert(MI == 32 || MI == 16, "32x32x16 or 16x16x32 matrix instruction");
    static_assert(KGROUPS == 1 || NWG * FM * FN * AV * 64 * 4 <= STAGES * (BM + BN) * BK * 2,
                  "the k-groups' sums are combined in the LDS ring");
    static_assert(BK == 32 || BK == 64 || BK == 128, "BK must be 32, 64 or 128");
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must be a multiple of the instruction tile");
    static_assert(KS >= 1, "a K tile holds at least one instruction's K");
    static_assert(STAGES >= 2 && STAGES <= 5, "2..5 LDS stages");
    static_assert(NL * (STAGES - 1) < 64, "vmcnt is 6 bits");
    static_assert(STAGGER == 0 || (STAGGER >= 2 && STAGGER <= 64), "K order: 0, or 2..64 start offsets");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
};

// Copies and the waits for them are issued through inline asm, so the
// compiler neither tracks them nor inserts its own conservative "vmcnt(0)
// before any LDS read" waits (which would serialize the prefetch); the
// kernel accounts for them with explicit vmcnt waits.  The "memory" clobber
// keeps every compiler-visible memory access on its side of each copy, and
// volatile asm is not moved across other volatile asm or barriers, so the
// source order below is the issue order.

// Raw buffer descriptor in four scalar registers: 48-bit base, stride 0,
// num_records, gfx9-family data-format word.
__device__ __forceinline__ i32x4 make_rsrc4(const void *base)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{(int32_t)(uint32_t)p, (int32_t)(uint32_t)(p >> 32), kNumRecords, kRsrcWord3};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One wave instruction: lane l copies 16 bytes from rsrc at voff + soff into
// LDS at byte address lds_addr + 16*l.  M0 carries lds_addr; one wait state
// separates its write from the copy that reads it.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// The operand tile as it sits in memory: a window of `row_left` rows (capped
// by the tile) of the stored matrix, `chunk_left` elements wide, starting at
// `origin`, rows `ld` elements apart.  For a K-contiguous tile the rows are
// M rows or N columns and the width runs along K; otherwise the rows are k
// values and the width runs along M or N.
struct TileSrc {
    const uint16_t *origin;
    int64_t ld;
    int64_t row_left;
    int64_t chunk_left;
};

// Copy number i (0 .. T::PW-1) of this wave for one operand tile: LDS row
// r = RPI*j + lane/CH with j = i*NW + wave, physical chunk lane%CH, logical
// chunk (lane%CH) ^ swz(r).
template <class T>
__device__ __forceinline__ void copy_slot(int i, int wave, int lane, i32x4 rs, const TileSrc &src,
                                          uint32_t region)
{
    const int j = i * T::NWAVES + wave;
    const int rl = lane / T::CH;
    const int r = T::RPI * j + rl;
    const int c = (lane % T::CH) ^ T::swz(r);
    const bool ok = r < src.row_left && 8 * c + 8 <= src.chunk_left;
    const uint32_t voff = (uint32_t)((rl * src.ld + 8 * c) * 2);
    dma16(rs, region + j * 1024, ok ? voff : kOOB, (uint32_t)(T::RPI * j * src.ld * 2));
}

// Register fill of the vectors of one operand tile that straddle the end of
// a row (the copies wrote zeros there): element loads, zero past the edge,
// written to the slot the copy would have filled.  Runs after this thread's
// copies for the tile have landed.
template <class T>
__device__ __forceinline__ void fill_tile(int wave, int lane, const TileSrc &src, lds_u8 *region)
{
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src.origin);
    // the tile's extent, clipped to the tile in 32 bits (both are positive)
    const int rows = (int)(src.row_left < T::ROWS ? src.row_left : T::ROWS);
    const int elems = (int)(src.chunk_left < 8 * T::CH ? src.chunk_left : 8 * T::CH);
    // This path runs only for tiles at a ragged edge.  The empty asm makes
    // the lane index opaque here, so the per-lane addressing below is
    // computed when the path runs instead of being hoisted out of the
    // kernel's main loop, where it would hold registers the whole time.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < T::PW; ++i) {
        const int j = i * T::NWAVES + wave;
        const int r = T::RPI * j + ln / T::CH;
        const int c = (ln % T::CH) ^ T::swz(r);
        const int left = elems - 8 * c;
        const int nv = r >= rows ? 0 : (left >= 8 ? 8 : (left <= 0 ? 0 : left));
        if (nv > 0 && nv < 8) {
            const uint32_t off = (uint32_t)((r * src.ld + 8 * c) * 2);
            *(lds_u32x4 *)(region + j * 1024 + ln * 16) = load8_partial(rs, off, nv);
        }
    }
}

// Does a tile with this many elements along its rows leave a partial vector?
template <class T>
__device__ __forceinline__ bool has_partial(int64_t chunk_left)
{
    return chunk_left < 8 * T::CH && (chunk_left & 7) != 0;
}

// Per-lane operand read addressing for a wave whose part of the operand
// starts at outer index `w_off` (wm*WTM for A, wn*WTN for B), for the
// 32x32x16 (MI = 32) or 16x16x32 (MI = 16) matrix instruction.
template <class T, int MI = 32>
struct OpReader {
    int base;    // byte offset of this lane's first read within the region
    int sw;      // swizzle of this lane's rows
    int col;     // outer-contiguous: this lane's first column

    __device__ __forceinline__ OpReader(int w_off, int lane)
    {
        if constexpr (T::K_CONTIG) {
            const int row = w_off + (lane & (MI - 1));
            sw = T::swz(row);
            base = row * T::ROWB;
            col = 0;
        } else if constexpr (MI == 32) {
            // group g = lane/16, index q = lane%16: rows 8*(g/2) + q/4 (+ 16*ks
            // + 4*h, which leave the swizzle unchanged), columns 16*(g%2) + 4*(q%4)
            const int g = lane >> 4, q = lane & 15;
            const int row_l = 8 * (g >> 1) + (q >> 2);
            sw = T::swz(row_l);
            base = row_l * T::ROWB;
            col = w_off + 16 * (g & 1) + 4 * (q & 3);
        } else {
            // rows 8*g + q/4 (+ 32*ks + 4*h, which leave the swizzle
            // unchanged), columns 4*(q%4)
            const int g = lane >> 4, q = lane & 15;
            const int row_l = 8 * g + (q >> 2);
            sw = T::swz(row_l);
            base = row_l * T::ROWB;
            col = w_off + 4 * (q & 3);
        }
    }

    // The 8 K-consecutive values lane l contributes to MFMA operand f of
    // k-step ks: outer index (w_off + MI*f + l%MI), k = KD*ks + 8*(l/MI) + 0..7
    // with KD = 16 (MI = 32) or 32 (MI = 16).
    __device__ __forceinline__ half8 read(const lds_u8 *region, int ks, int f, int lane) const
    {
        constexpr int KD = MI == 32 ? 16 : 32;
        if constexpr (T::K_CONTIG) {
            const int off = base + f * MI * T::ROWB + ((((KD / 8) * ks + lane / MI) ^ sw) * 16);
            return __builtin_bit_cast(half8, *(const lds_u32x4 *)(region + off));
        } else {
            const int c = col + MI * f;
            const lds_u8 *p0 = region + base + KD * ks * T::ROWB + (((c >> 3) ^ sw) * 16) + (c & 7) * 2;
            const fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) fp16x4 *)p0);
            const fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                (__attribute__((address_space(3))) fp16x4 *)(p0 + 4 * T::ROWB));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
};

template <class Cfg, bool NT_STORES = true>
__global__ void __launch_bounds__(Cfg::NT)
gemm_pipe(GemmArgs args_in)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, S = Cfg::STAGES;
    constexpr int FM = Cfg::FM, FN = Cfg::FN, KS = Cfg::KS;
    constexpr int APW = Cfg::APW, BPW = Cfg::BPW, NL = Cfg::NL, NCOPY = Cfg::NCOPY;
    using TA = typename Cfg::TA;
    using TB = typename Cfg::TB;
    constexpr bool A_ROW = Cfg::LAYOUT_A == kRowMajor;
    constexpr bool B_ROW = Cfg::LAYOUT_B == kRowMajor;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_BYTES];
    lds_u8 *const lds = (lds_u8 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
#ifdef MPGEMM_TIMELINE
    __shared__ uint64_t timeline[kTimelineSlots];
    if (tid == 0) {
        timeline[0] = __builtin_amdgcn_s_memrealtime();
        timeline[1] = __builtin_amdgcn_s_memtime();
        for (int i = 2; i < kTimelineSlots; ++i)
            timeline[i] = 0;
    }
#endif
    // timeline build: shader-clock stamp of tile t's publish (no code otherwise)
    auto stamp_tile = [&](int64_t t) __attribute__((always_inline)) {
#ifdef MPGEMM_TIMELINE
        if (tid == 0 && t < kTimelineTiles)
            timeline[2 + t] = __builtin_amdgcn_s_memtime();
#else
        (void)t;
#endif
    };
    const int lane = tid & 63;
    // wave index, made explicitly wave-uniform so everything derived from it
    // (copy offsets, M0) stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kgroup = wave / Cfg::NWG;              // 0 unless k-groups
    const int wl = wave - kgroup * Cfg::NWG;         // wave within its k-group
    const int wm = wl / Cfg::WAVES_N;
    const int wn = wl % Cfg::WAVES_N;
    const int ks0 = kgroup * Cfg::KSL;               // this group's first k-step of a tile

    // Split-K: this workgroup's K range and partial-sum destination; the rest
    // of the kernel sees an ordinary product over that range.
    GemmArgs args = args_in;
    int bid = blockIdx.x, nb = gridDim.x;
    if (args.splits > 1) {
        const int ntiles = args.tiles_m * args.tiles_n;
        const int split = bid / ntiles;
        bid -= split * ntiles;
        nb = ntiles;
        const int64_t k0 = (int64_t)split * args.k_split;
        const int64_t klen = args.K - k0 < args.k_split ? args.K - k0 : args.k_split;
        args.A += A_ROW ? k0 : k0 * args.lda;
        args.B += B_ROW ? k0 * args.ldb : k0;
        args.K = klen > 0 ? klen : 0;
        args.C = args.ws + (int64_t)split * args.M * args.N;
        args.ldc = args.N;
        args.alpha = 1.0f;
        args.beta = 0.0f;
        args.bias = nullptr;
    }

    int tm, tn;
    tile_coords(bid, nb, args.tiles_n, args.tiles_m, args.group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    // K tail: the copy loop covers the largest multiple of 8 of K, so every
    // 16-byte vector it copies is either whole or wholly past the edge; the
    // last K % 8 values are one more matrix-instruction step whose operands
    // come straight from memory (see tail_load).
    const int ktail = (int)(args.K & 7);
    const int64_t K = args.K - ktail;
    const int64_t lda = args.lda, ldb = args.ldb;
    const int64_t rows_left = args.M - m0;  // > 0
    const int64_t cols_left = args.N - n0;  // > 0

    // K tile t of the loop is K tile (t + koff) mod num_kt of the matrices
    // (see PipeCfg::STAGGER).  Only the order of the K tiles changes; the K
    // tail stays the last step.
    const int64_t num_kt = (K + BK - 1) / BK;
    int64_t koff = 0;
    if constexpr (Cfg::STAGGER != 0) {
        const int spread = num_kt < Cfg::STAGGER ? (int)num_kt : Cfg::STAGGER;
        koff = spread > 1 ? (tm + tn) % spread : 0;
    }
    auto kmem = [&](int64_t t) __attribute__((always_inline)) {
        if constexpr (Cfg::STAGGER == 0)
            return t;
        else
            return t + koff < num_kt ? t + koff : t + koff - num_kt;
    };

    // The A and B tiles of K tile t as windows of the stored matrices.
    auto src_a = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t k0 = kmem(t) * BK;
        if constexpr (A_ROW)
            return TileSrc{args.A + m0 * lda + k0, lda, rows_left, K - k0};
        else
            return TileSrc{args.A + k0 * lda + m0, lda, K - k0, rows_left};
    };
    auto src_b = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t k0 = kmem(t) * BK;
        if constexpr (B_ROW)
            return TileSrc{args.B + k0 * ldb + n0, ldb, K - k0, cols_left};
        else
            return TileSrc{args.B + n0 * ldb + k0, ldb, cols_left, K - k0};
    };

    // ---- copies of one K tile into one ring buffer, issued a few at a time
    TileSrc cpa{}, cpb{};
    uint32_t copy_region = 0;  // LDS byte address of the buffer being filled
    bool copy_live = false;
    i32x4 rsA, rsB;
    auto begin_copies = [&](int64_t t, int buf) __attribute__((always_inline)) {
        copy_region = lds_base + buf * Cfg::STAGE_BYTES;
        copy_live = t < (K + BK - 1) / BK;
        cpa = src_a(t);
        cpb = src_b(t);
        rsA = make_rsrc4(cpa.origin);
        rsB = make_rsrc4(cpb.origin);
    };
    // copy number q (0 .. NCOPY-1) of the current tile
    auto copy_one = [&](int q) __attribute__((always_inline)) {
        if (!copy_live)
            return;
        if (q < APW)
            copy_slot<TA>(q, wave, lane, rsA, cpa, copy_region);
        else
            copy_slot<TB>(q - APW, wave, lane, rsB, cpb, copy_region + Cfg::A_BYTES);
    };

    // Register fill of the vectors that straddle a row end, after this
    // thread's copies of tile kt have landed.
    auto fill = [&](int64_t kt, int buf) __attribute__((always_inline)) {
        lds_u8 *const sbase = lds + buf * Cfg::STAGE_BYTES;
        const TileSrc a = src_a(kt), b = src_b(kt);
        if (has_partial<TA>(a.chunk_left))
            fill_tile<TA>(wave, lane, a, sbase);
        if (has_partial<TB>(b.chunk_left))
            fill_tile<TB>(wave, lane, b, sbase + Cfg::A_BYTES);
    };
    auto needs_fill = [&](int64_t kt) __attribute__((always_inline)) {
        return has_partial<TA>(src_a(kt).chunk_left) || has_partial<TB>(src_b(kt).chunk_left);
    };

    // ---- operand reads -----------------------------------------------------
    const OpReader<TA, Cfg::MI> rd_a(wm * Cfg::WTM, lane);
    const OpReader<TB, Cfg::MI> rd_b(wn * Cfg::WTN, lane);
    // With the 16x16x32 instruction a wave holds twice as many operand
    // registers per k-step; A operand f is then kept in one register set and
    // reloaded for the next k-step right after the MFMAs of group f have
    // issued (still a whole k-step ahead of its use).
    constexpr bool ROLL_A = Cfg::MI == 16;
    half8 ra[ROLL_A ? 1 : 2][FM], rb[2][FN];
    auto read_a = [&](int buf, int ks, int set, int f) __attribute__((always_inline)) {
        ra[ROLL_A ? 0 : set][f] = rd_a.read(lds + buf * Cfg::STAGE_BYTES, ks, f, lane);
    };
    auto read_b = [&](int buf, int ks, int set, int f) __attribute__((always_inline)) {
        rb[set][f] = rd_b.read(lds + buf * Cfg::STAGE_BYTES + Cfg::A_BYTES, ks, f, lane);
    };
    // reads for one group: A operand f (if f < FM) and the B operands
    // assigned to that group (FN spread over FM groups)
    auto read_group = [&](int buf, int ks, int set, int grp) __attribute__((always_inline)) {
        read_a(buf, ks, set, grp);
#pragma unroll
        for (int f = 0; f < FN; ++f)
            if (f % FM == grp)
                read_b(buf, ks, set, f);
    };

    // ---- K tail operands.  The instruction sums over all of its K
    // positions, so where a tail value sits among them does not matter as
    // long as A and B put it in the same place: tail value j (0 <= j <
    // ktail <= 7) goes to lane group g = j % G (lanes MI*g .. MI*g + MI - 1,
    // G = 64 / MI groups) at element j / G of the group's 8, the other
    // elements stay zero.  Every lane then loads NS = ceil(7 / G) values (2
    // for 16x16x32, 4 for 32x32x16) instead of one lane group loading all 8.
    // Values at and past the true K, and past the M or N edge, read as zero.
    // 2-byte buffer loads; the 32-bit offsets stay within the stage span the
    // host checks.  With small wave tiles the loads go out before the ring
    // fill, the oldest memory operations of the kernel, so the copy waits
    // cover them and their latency hides under the K loop; large wave tiles,
    // which have no registers to spare across the loop, issue them after it.
    constexpr bool TAIL_EARLY = (FM + FN) * 4 <= 16;
    constexpr int TG = 64 / Cfg::MI;
    constexpr int TNS = (7 + TG - 1) / TG;
    half8 ta[FM], tb[FN];
    auto tail_load = [&]() __attribute__((always_inline)) {
        constexpr int MI = Cfg::MI;
        const int li = lane & (MI - 1);
        const int g = lane / MI;
        const int ld_a = (int)lda, ld_b = (int)ldb;
        const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(args.A + (A_ROW ? m0 * lda + K : K * lda + m0));
        const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(args.B + (B_ROW ? K * ldb + n0 : n0 * ldb + K));
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const int r = wm * Cfg::WTM + MI * f + li;
            const bool r_ok = r < rows_left;
            uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < TNS; ++e) {
                const int k = TG * e + g;
                const uint32_t off = (uint32_t)((A_ROW ? r * ld_a + k : k * ld_a + r) * 2);
                h[e] = __builtin_amdgcn_raw_buffer_load_b16(rs_a, (r_ok && k < ktail) ? off : kOOB, 0, 0);
            }
            ta[f] = __builtin_bit_cast(half8, u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]),
                                                    pack2(h[6], h[7])});
        }
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const int c = wn * Cfg::WTN + MI * f + li;
            const bool c_ok = c < cols_left;
            uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < TNS; ++e) {
                const int k = TG * e + g;
                const uint32_t off = (uint32_t)((B_ROW ? k * ld_b + c : c * ld_b + k) * 2);
                h[e] = __builtin_amdgcn_raw_buffer_load_b16(rs_b, (c_ok && k < ktail) ? off : kOOB, 0, 0);
            }
            tb[f] = __builtin_bit_cast(half8, u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]),
                                                    pack2(h[6], h[7])});
        }
    };
    if constexpr (TAIL_EARLY) {
        if (ktail > 0)
            tail_load();
    }

    constexpr int AV = Cfg::AV;
    using AccT = typename std::conditional<Cfg::MI == 32, floatx16, floatx4>::type;
    AccT acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = AccT{0};

    auto mfma_group = [&](int set, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (Cfg::MI == 32)
                acc[i][j] = mfma32<Cfg::IN>(ra[set][i], rb[set][j], acc[i][j]);
            else
                acc[i][j] = mfma16<Cfg::IN>(ra[ROLL_A ? 0 : set][i], rb[set][j], acc[i][j]);
        }
    };

    // Make tile t (in buffer buf) visible to the workgroup: this thread's
    // copies of tile t have landed (the `newer` whole tiles issued after it
    // may still be in flight), registers fill what the copies could not,
    // then the barrier.
    auto publish = [&](int64_t t, int buf, int newer) __attribute__((always_inline)) {
        if (needs_fill(t)) {
            wait_vmcnt<0>();
            fill(t, buf);
        } else if (newer <= 0) {
            wait_vmcnt<0>();
        } else if (newer == 1) {
            wait_vmcnt<NL>();
        } else if (newer == 2) {
            wait_vmcnt<(S > 2 ? 2 : 1) * NL>();
        } else if (newer == 3) {
            wait_vmcnt<(S > 3 ? 3 : 1) * NL>();
        } else {
            wait_vmcnt<(S > 4 ? 4 : 1) * NL>();
        }
        __syncthreads();
    };
    // the copies of the current copy tile that belong to window position p
    auto copy_slice = [&](int p) __attribute__((always_inline)) {
        constexpr int W = Cfg::COPY_WINDOW;
#pragma unroll
        for (int c = 0; c < NCOPY; ++c)
            if (c >= (p * NCOPY + W - 1) / W && c < ((p + 1) * NCOPY + W - 1) / W)
                copy_one(c);
    };

    const int64_t num_k = (K + BK - 1) / BK;
    if (num_k > 0) {
        // the whole ring: tiles 0 .. S-1
#pragma unroll
        for (int t = 0; t < S; ++t) {
            begin_copies(t, t);
#pragma unroll
            for (int c = 0; c < NCOPY; ++c)
                copy_one(c);
        }
        publish(0, 0, (int)(num_k - 1 < S - 1 ? num_k - 1 : S - 1));
        stamp_tile(0);
#pragma unroll
        for (int grp = 0; grp < FM; ++grp)
            read_group(0, ks0, 0, grp);
    }
    int buf = 0;
    for (int64_t kt = 0; kt < num_k; ++kt) {
        const int nbuf = (buf + 1 == S) ? 0 : buf + 1;

        // ks counts this k-group's k-steps of the tile (all of them without
        // k-groups); the LDS rows read are those of k-step ks0 + ks
#pragma unroll
        for (int ks = 0; ks < Cfg::KSL; ++ks) {
            const int set = ks & 1;
            const bool last = ks + 1 == Cfg::KSL;
            if (last && kt + 1 < num_k) {
                // tiles kt+2 .. kt+S-1 may still be in flight
                const int64_t newer = num_k - 2 - kt;
                publish(kt + 1, nbuf, (int)(newer < S - 2 ? newer : S - 2));
                stamp_tile(kt + 1);
            }
            if (last)
                begin_copies(kt + S, buf);
            // All operand reads for the next k-step go out first, a whole
            // k-step (16 MFMAs per wave) ahead of their use; the scheduling
            // barriers keep the compiler from sinking them next to their uses.
            // (Rolling A: only the B reads go out here.)
#pragma unroll
            for (int grp = 0; grp < FM; ++grp) {
                if constexpr (ROLL_A) {
#pragma unroll
                    for (int f = 0; f < FN; ++f)
                        if (f % FM == grp) {
                            if (!last)
                                read_b(buf, ks0 + ks + 1, set ^ 1, f);
                            else if (kt + 1 < num_k)
                                read_b(nbuf, ks0, set ^ 1, f);
                        }
                } else {
                    if (!last)
                        read_group(buf, ks0 + ks + 1, set ^ 1, grp);
                    else if (kt + 1 < num_k)
                        read_group(nbuf, ks0, set ^ 1, grp);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int grp = 0; grp < FM; ++grp) {
                mfma_group(set, grp);
                if constexpr (ROLL_A) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (!last)
                        read_a(buf, ks0 + ks + 1, set ^ 1, grp);
                    else if (kt + 1 < num_k)
                        read_a(nbuf, ks0, set ^ 1, grp);
                }
                // The last k-step opens the window of tile kt+S; the others
                // continue that of tile kt+S-1, which the ring fill issued
                // whole when kt == 0.
                if (last)
                    copy_slice(grp);
                else if (kt > 0)
                    copy_slice(FM + ks * FM + grp);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        buf = nbuf;
    }

    // ---- k-groups: group g > 0 hands its sums to group 0 through LDS
    if constexpr (Cfg::KGROUPS > 1) {
        static_assert(Cfg::KGROUPS == 2, "two k-groups");
        float *const xfer = (float *)smem;
        __syncthreads();  // every wave is past its last read of the ring
        if (kgroup == 1) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < AV; ++v)
                        xfer[(((wl * FM + i) * FN + j) * AV + v) * 64 + lane] = acc[i][j][v];
        }
        __syncthreads();
        if (kgroup == 1)
            return;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < AV; ++v)
                    acc[i][j][v] += xfer[(((wl * FM + i) * FN + j) * AV + v) * 64 + lane];
    }

    // ---- K tail: one more instruction step on the tail operands
    if (ktail > 0) {
        if constexpr (!TAIL_EARLY)
            tail_load();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (Cfg::MI == 32)
                    acc[i][j] = mfma32<Cfg::IN>(ta[i], tb[j], acc[i][j]);
                else
                    acc[i][j] = mfma16<Cfg::IN>(ta[i], tb[j], acc[i][j]);
            }
    }

#ifdef MPGEMM_TIMELINE
    if (tid == 0)
        timeline[44] = __builtin_amdgcn_s_memtime();
#endif

    // ---- epilogue: C = alpha*acc + beta*C through buffer stores whose
    // out-of-range offsets the hardware drops (and loads read as zero).
    // The stores' cache policy is the kernel's NT_STORES: non-temporal, so
    // C does not evict the A and B panels other workgroups are still
    // streaming through the caches, or plain, so that a large burst of C (or
    // rows that start mid-line) is absorbed by the caches; the host picks
    // the variant per call.
    constexpr int32_t kPolicy = NT_STORES ? kStoreNT : 0;
    const int64_t wrow0 = m0 + wm * Cfg::WTM;
    const int64_t wcol0 = n0 + wn * Cfg::WTN;
    const int64_t wrows = args.M - wrow0;
    const int64_t wcols = args.N - wcol0;
    if (wrows > 0 && wcols > 0) {
        const __amdgpu_buffer_rsrc_t rsC = make_rsrc(args.C + wrow0 * args.ldc + wcol0);
        const int ldc = (int)args.ldc;
        const float alpha = args.alpha, beta = args.beta;
        // accumulator v of instruction tile (i, j) holds row
        // MI*i + rl + (MI == 32 ? 8*(v/4) + v%4 : v), column MI*j + cl
        constexpr int MI = Cfg::MI;
        const int cl = lane & (MI - 1);
        const int rl = 4 * (lane / MI);
        if constexpr (MI == 16 && FN % 2 == 0) {
            // Full-line stores.  Accumulator v of lane l holds row 4*(l/16)
            // + v of a 16-column instruction tile, so one store covers 64
            // bytes of each of four rows (half lines), which cost about a
            // fifth more write traffic.  Tiles 2p and 2p+1 are adjacent:
            // swapping the odd 16-lane rows of tile 2p's value with the even
            // rows of tile 2p+1's (v_permlane16_swap) leaves lane l with row
            // v + 8*(l/32) (first value) and 4 + v + 8*(l/32) (second) of
            // column 32p + l%32, so each store writes two whole 128-byte
            // lines.
            const int cp = lane & 31;
            const int rp = 8 * (lane >> 5);
            float bp[FN / 2];
#pragma unroll
            for (int p = 0; p < FN / 2; ++p)
                bp[p] = 0.0f;
            if (args.bias) {
                const __amdgpu_buffer_rsrc_t rsBias = make_rsrc(args.bias + wcol0);
#pragma unroll
                for (int p = 0; p < FN / 2; ++p) {
                    const int c = 32 * p + cp;
                    bp[p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          rsBias, c < wcols ? (uint32_t)(c * 4) : kOOB, 0, 0));
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int p = 0; p < FN / 2; ++p) {
                    const int c = 32 * p + cp;
                    const bool c_ok = c < wcols;
                    uint32_t off[2][AV];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int v = 0; v < AV; ++v) {
                            const int r = MI * i + 4 * h + v + rp;
                            off[h][v] = (c_ok && r < wrows) ? (uint32_t)((r * ldc + c) * 4) : kOOB;
                        }
                    float cin[2][AV];
                    if (beta != 0.0f) {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int v = 0; v < AV; ++v)
                                cin[h][v] = __builtin_bit_cast(
                                    float, __builtin_amdgcn_raw_buffer_load_b32(rsC, off[h][v], 0, 0));
                    }
#pragma unroll
                    for (int v = 0; v < AV; ++v) {
                        // (scalar copies first: a bit cast applied to a vector
                        // element directly reads element 0 with this compiler)
                        const float x0 = acc[i][2 * p][v], x1 = acc[i][2 * p + 1][v];
                        const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x0),
                                                                         __builtin_bit_cast(uint32_t, x1), false,
                                                                         false);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            float val = alpha * __builtin_bit_cast(float, (uint32_t)sw[h]);
                            if (beta != 0.0f)
                                val = __builtin_fmaf(beta, cin[h][v], val);
                            if (args.bias)
                                val += bp[p];
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rsC,
                                                                  off[h][v], 0, kPolicy);
                        }
                    }
                }
            }
        } else {
            // the bias of each of this lane's FN columns (0 past the last column)
            float bv[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bv[j] = 0.0f;
            if (args.bias) {
                const __amdgpu_buffer_rsrc_t rsBias = make_rsrc(args.bias + wcol0);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int c = MI * j + cl;
                    bv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          rsBias, c < wcols ? (uint32_t)(c * 4) : kOOB, 0, 0));
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int c = MI * j + cl;
                    const bool c_ok = c < wcols;
                    uint32_t off[AV];
#pragma unroll
                    for (int v = 0; v < AV; ++v) {
                        const int r = MI * i + rl + (MI == 32 ? 8 * (v >> 2) + (v & 3) : v);
                        off[v] = (c_ok && r < wrows) ? (uint32_t)((r * ldc + c) * 4) : kOOB;
                    }
                    // With beta != 0 all of the tile's C loads go out before its
                    // first store: the loads and stores share a buffer, so the
                    // compiler keeps them in program order, and loading each
                    // element just before its store would serialize the loads.
                    float cin[AV];
                    if (beta != 0.0f) {
#pragma unroll
                        for (int v = 0; v < AV; ++v)
                            cin[v] = __builtin_bit_cast(
                                float, __builtin_amdgcn_raw_buffer_load_b32(rsC, off[v], 0, 0));
                    }
#pragma unroll
                    for (int v = 0; v < AV; ++v) {
                        float val = alpha * acc[i][j][v];
                        if (beta != 0.0f)
                            val = __builtin_fmaf(beta, cin[v], val);
                        if (args.bias)
                            val += bv[j];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rsC, off[v], 0,
                                                              kPolicy);
                    }
                }
            }
        }
    }
#ifdef MPGEMM_TIMELINE
    if (tid == 0) {
        timeline[45] = __builtin_amdgcn_s_memtime();
        timeline[46] = __builtin_amdgcn_s_memrealtime();
        uint32_t hw_id, xcc_id;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw_id));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc_id));
        timeline[47] = ((uint64_t)xcc_id << 32) | hw_id;
        timeline[43] = (uint64_t)num_k;
        if (blockIdx.x < kTimelineWgs)
            for (int i = 0; i < kTimelineSlots; ++i)
                g_timeline[(int64_t)blockIdx.x * kTimelineSlots + i] = timeline[i];
    }
#endif
}

// ---------------------------------------------------------------------------
// Narrow kernel: N <= 16 (one 16-column instruction tile), A row-major
// ---------------------------------------------------------------------------
// A product with at most 16 columns is a stream over A (the "skinny" shape
// of the capstone gate): block tiles wide enough to amortize an LDS ring
// would mostly multiply zeros, and an under-filled grid leaves the memory
// system idle.  Each workgroup takes 16 rows of C; its 8 waves split the K
// range into 8 slices.  A wave streams its slice of A straight from memory
// into operand registers (lane l: row l % 16, 8 consecutive k at
// 8*(l/16) of each 32-deep step, one 16-byte buffer load; out-of-range rows
// and K read zero) and loads B beside it: a column-major B with one 16-byte
// load of the operand's 8 k values; a row-major B with one 16-byte load of
// 8 consecutive columns of one k row per lane (the k-step's 32 x 16 values
// in one instruction; columns past N only reach output columns that are
// never stored), turned into operand layout through a 1 KiB LDS
// slot of the wave's own and the transposing LDS read.  It accumulates a
// 16x16 partial tile on the 16x16x32 instruction, with the loads DEPTH
// k-steps ahead of their use (two loads per k-step except where a row-major
// B vector would run past B's last element, so the 6-bit load counter covers
// deep rings).  As in the
// pipelined kernel the main range covers the largest multiple of 8 of K and
// the last K % 8 values are one more step (wave 0).  The 8 partial tiles
// are summed through LDS in ascending slice order (run-to-run identical),
// then wave 0 applies alpha, beta and the bias and stores the tile.
// 32-bit buffer offsets: the host checks that 16 rows of A, the K (or 16)
// stored rows of B and 16 rows of C fit them.
template <int IN, int LB, int DEPTH>
__global__ void __launch_bounds__(512)
gemm_narrow(GemmArgs args)
{
    constexpr bool B_ROW = LB == 0;
    __shared__ floatx4 part[8][64];
    __shared__ u32x4 bslot[8][64];  // row-major B: each wave's transpose slot
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t M = args.M, N = args.N;
    const int ktail = (int)(args.K & 7);
    const int64_t Km = args.K - ktail;
    const int r = lane & 15;          // A row / B column of this lane
    const int kq = 8 * (lane >> 4);   // this lane's 8 k values within a step
    const bool r_ok = m0 + r < M;
    const bool n_ok = r < N;
    const int lda = (int)args.lda, ldb = (int)args.ldb;
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(args.A + m0 * args.lda);
    const __amdgpu_buffer_rsrc_t rsB = make_rsrc(args.B);

    // this wave's k-steps [s0, s1) of the main range
    const int64_t steps = (Km + 31) / 32;
    const int64_t per = (steps + 7) / 8;
    const int64_t s0 = wave * per;
    const int64_t s1 = s0 + per < steps ? s0 + per : steps;

    // row-major B: lane j loads columns 8*(j%2)..+7 of k row j/2 of the step
    // with one 16-byte load.  Values it brings in from columns at or past N
    // (row padding, or the next row) land in operand columns >= N, which
    // only feed output columns >= N: those are never stored, so they need
    // no zeroing.  Only a vector that would run past B's last stored element
    // (kr*ldb + bn + 7 > (K-1)*ldb + N-1: the last rows of a packed B
    // narrower than 8 columns) is loaded element by element instead.
    const int bk = lane >> 1, bn = 8 * (lane & 1);
    const bool b_full = bn + 8 <= N;
    const bool b_some = bn < N;
    // index of B's last stored element, (K-1)*ldb + N-1: below 2^30, since
    // the host checks that B's stored rows span fewer than 2^31 bytes
    const int b_last = (int)((args.K - 1) * args.ldb + N - 1);
    u32x4 ra[DEPTH], rb[DEPTH];
    auto issue = [&](int d, int64_t s) __attribute__((always_inline)) {
        const int64_t k = 32 * s + kq;
        const bool k_ok = k + 8 <= Km;
        ra[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rsA, (r_ok && k_ok) ? (uint32_t)((r * lda + (int)k) * 2) : kOOB, 0, 0));
        if constexpr (B_ROW) {
            const int64_t kr = 32 * s + bk;
            // used only when row kr is in range (within the span the host checks)
            const uint32_t off = (uint32_t)((kr * args.ldb + bn) * 2);
            if (b_full || !b_some || kr >= Km || (int)kr * ldb + bn + 7 <= b_last) {
                rb[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rsB, (b_some && kr < Km) ? off : kOOB, 0, 0));
            } else {
                // the vector would run past B's last element: element by element
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = __builtin_amdgcn_raw_buffer_load_b16(rsB, bn + e < N ? off + 2u * e : kOOB, 0, 0);
                rb[d] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
            }
        } else {
            rb[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rsB, (n_ok && k_ok) ? (uint32_t)((r * ldb + (int)k) * 2) : kOOB, 0, 0));
        }
    };
    // the B operand of the step in register set d: lane l needs k = 8*(l/16)
    // + 0..7 of column l % 16.  Row-major: the 32 k rows of 32 bytes go into
    // the wave's slot (lane j at byte 16*j = row j/2, half j%2), and two
    // transposing reads give lane 16*g + i the 4 + 4 values of column i at
    // rows 8*g + 0..3 and 8*g + 4..7 (in each 16-lane group, lane i's slot
    // t takes element i%4 of the 8 bytes addressed by lane 4*t + i/4, which
    // addresses row 8*g + t at column 4*(i/4)).  The slot is the wave's own
    // and LDS operations of one wave complete in order, so no barrier.
    auto b_operand = [&](int d) __attribute__((always_inline)) {
        if constexpr (B_ROW) {
            *(lds_u32x4 *)&bslot[wave][lane] = rb[d];
            const int g = lane >> 4, q = lane & 15;
            const lds_u8 *p0 = (const lds_u8 *)&bslot[wave][0] + (8 * g + (q >> 2)) * 32 + 8 * (q & 3);
            const fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) fp16x4 *)p0);
            const fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                (__attribute__((address_space(3))) fp16x4 *)(p0 + 4 * 32));
            return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return __builtin_bit_cast(half8, rb[d]);
        }
    };

    floatx4 acc = floatx4{0};
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (s0 + d < s1)
            issue(d, s0 + d);
    for (int64_t s = s0; s < s1; s += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (s + d < s1) {
                const half8 a = __builtin_bit_cast(half8, ra[d]);
                acc = mfma16<IN>(a, b_operand(d), acc);
                if (s + d + DEPTH < s1)
                    issue(d, s + d + DEPTH);
            }
        }
    }

    // the last K % 8 values: lane l holds k = Km + kq + 0..7, zero at and past K
    if (wave == 0 && ktail > 0) {
        uint32_t ha[8], hb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = kq + e;
            const bool ok = k < ktail;
            const int kk = (int)Km + k;
            ha[e] = __builtin_amdgcn_raw_buffer_load_b16(rsA, (r_ok && ok) ? (uint32_t)((r * lda + kk) * 2) : kOOB,
                                                         0, 0);
            hb[e] = __builtin_amdgcn_raw_buffer_load_b16(
                rsB, (n_ok && ok) ? (uint32_t)((B_ROW ? kk * ldb + r : r * ldb + kk) * 2) : kOOB, 0, 0);
        }
        const half8 a = __builtin_bit_cast(half8, u32x4{pack2(ha[0], ha[1]), pack2(ha[2], ha[3]),
                                                        pack2(ha[4], ha[5]), pack2(ha[6], ha[7])});
        const half8 b = __builtin_bit_cast(half8, u32x4{pack2(hb[0], hb[1]), pack2(hb[2], hb[3]),
                                                        pack2(hb[4], hb[5]), pack2(hb[6], hb[7])});
        acc = mfma16<IN>(a, b, acc);
    }

    // sum the 8 partial tiles in ascending slice order
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0)
        return;
    floatx4 sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w)
        sum += part[w][lane];

    // epilogue: accumulator v of lane l holds row 4*(l/16) + v, column l % 16
    const __amdgpu_buffer_rsrc_t rsC = make_rsrc(args.C + m0 * args.ldc);
    const int ldc = (int)args.ldc;
    const int col = lane & 15;
    const bool c_ok = col < N;
    float bv = 0.0f;
    if (args.bias && c_ok)
        bv = args.bias[col];
    uint32_t off[4];
    float cin[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int row = 4 * (lane >> 4) + v;
        off[v] = (c_ok && m0 + row < M) ? (uint32_t)((row * ldc + col) * 4) : kOOB;
        cin[v] = 0.0f;
    }
    if (args.beta != 0.0f) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            cin[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsC, off[v], 0, 0));
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float val = args.alpha * sum[v];
        if (args.beta != 0.0f)
            val = __builtin_fmaf(args.beta, cin[v], val);
        if (args.bias)
            val += bv;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rsC, off[v], 0, kStoreNT);
    }
}

}  // namespace mpg
