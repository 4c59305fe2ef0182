// mpgemm.hip -- host side of the gfx950 FP16-input / FP32-accumulate GEMM:
// argument validation, the tile-config factory, launches and the C ABI
// declared in include/mpgemm.h.
//
// The factory is the gfx950 form of the "kernel factory" of the
// "GEMM kernels 1-7 + Tensor Cores" visualizer (kernel 7: the host picks the
// tile shape per configuration): a small table of compiled block/wave tiles
// per input format and storage-order pair, chosen per shape so that the grid
// fills the 256 compute units, with the 64-bit direct kernel for whatever
// the tiled kernels' 32-bit buffer offsets cannot address.
#include "mpgemm.h"
#ifdef MPGEMM_TIMELINE
#include "mpgemm_timeline.h"
#endif

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.hpp"

namespace {

using mpg::GemmArgs;
using mpg::kColMajor;
using mpg::kInBF16;
using mpg::kInF16;
using mpg::kRowMajor;
using mpg::PipeCfg;

constexpr int kNumCu = 256;

// ---------------------------------------------------------------------------
// Config table
// ---------------------------------------------------------------------------
using launch_fn = hipError_t (*)(const GemmArgs &, dim3, hipStream_t);

// `launch` runs the entry with non-temporal C stores, `launch_plain` with
// plain ones (the same launch where the entry has one variant only).
struct Entry {
    mpgemm_config cfg;
    launch_fn launch;
    launch_fn launch_plain;
};

template <class Cfg, bool NT_STORES>
hipError_t launch_pipe(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((mpg::gemm_pipe<Cfg, NT_STORES>), grid, dim3(Cfg::NT), 0, s, a);
    return hipGetLastError();
}

template <int IN, int LB, int DEPTH>
hipError_t launch_narrow(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((mpg::gemm_narrow<IN, LB, DEPTH>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
}

template <int IN>
hipError_t launch_direct(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL(mpg::gemm_direct<IN>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <class Cfg>
constexpr Entry pipe_entry(int id)
{
    mpgemm_config c{};
    c.id = id;
    c.kind = MPGEMM_KIND_PIPE;
    c.bm = Cfg::BM;
    c.bn = Cfg::BN;
    c.bk = Cfg::BK;
    c.waves_m = Cfg::WAVES_M;
    c.waves_n = Cfg::WAVES_N;
    c.wave_m = Cfg::WTM;
    c.wave_n = Cfg::WTN;
    c.mfma_m = Cfg::MI;
    c.mfma_n = Cfg::MI;
    c.mfma_k = Cfg::KD;
    c.vec_a = 8;
    c.vec_b = 8;
    c.stages = Cfg::STAGES;
    c.threads = Cfg::NT;
    c.lds_bytes = Cfg::LDS_BYTES;
    c.grid = 0;
    c.layout_a = Cfg::LAYOUT_A;
    c.layout_b = Cfg::LAYOUT_B;
    c.in_type = Cfg::IN;
    c.k_groups = Cfg::KGROUPS;
    c.k_order = Cfg::STAGGER;
    c.c_stores = Cfg::BM == 256 ? 2 : 1;
    // 256x256 tiles also come with plain C stores (see nt_stores)
    launch_fn plain = &launch_pipe<Cfg, true>;
    if constexpr (Cfg::BM == 256)
        plain = &launch_pipe<Cfg, false>;
    return Entry{c, &launch_pipe<Cfg, true>, plain};
}

// N <= 16 with A row-major: 16 rows of C per workgroup, 8 waves over K.
template <int IN, int LB, int DEPTH>
constexpr Entry narrow_entry(int id)
{
    mpgemm_config c{};
    c.id = id;
    c.kind = MPGEMM_KIND_NARROW;
    c.bm = 16;
    c.bn = 16;
    c.bk = 32;
    c.waves_m = 1;
    c.waves_n = 1;
    c.wave_m = 16;
    c.wave_n = 16;
    c.mfma_m = 16;
    c.mfma_n = 16;
    c.mfma_k = 32;
    c.vec_a = 8;
    c.vec_b = 8;
    c.stages = DEPTH;   // k-steps of loads in flight per wave
    c.threads = 512;
    c.lds_bytes = 2 * 8 * 64 * 16;  // partial tiles + row-major B transpose slots
    c.layout_a = kRowMajor;
    c.layout_b = LB;
    c.in_type = IN;
    c.k_groups = 8;     // waves splitting K
    c.c_stores = 1;
    return Entry{c, &launch_narrow<IN, LB, DEPTH>, &launch_narrow<IN, LB, DEPTH>};
}

template <int IN>
constexpr Entry direct_entry(int id)
{
    mpgemm_config c{};
    c.id = id;
    c.kind = MPGEMM_KIND_DIRECT;
    c.bm = 64;
    c.bn = 64;
    c.bk = 16;
    c.waves_m = 2;
    c.waves_n = 2;
    c.wave_m = 32;
    c.wave_n = 32;
    c.mfma_m = 32;
    c.mfma_n = 32;
    c.mfma_k = 16;
    c.vec_a = 1;
    c.vec_b = 1;
    c.stages = 0;
    c.threads = 256;
    c.lds_bytes = 0;
    c.in_type = IN;
    c.k_groups = 1;
    return Entry{c, &launch_direct<IN>, &launch_direct<IN>};
}

constexpr Entry scale_entry(int id)
{
    mpgemm_config c{};
    c.id = id;
    c.kind = MPGEMM_KIND_SCALE;
    c.threads = 256;
    c.k_groups = 1;
    return Entry{c, nullptr, nullptr};
}

// The tile shapes the factory chooses from, for one input format and
// storage-order pair (entries base .. base+3):
//   big   256x256x64, 2 stages, 8 waves of 128x64 on 16x16x32: products
//         whose 256x256 tiles take at most a third of the 128x128 tiles'
//         rounds over the compute units (under the board's power limit this
//         instruction does 3-8% more work per joule than 32x32x16);
//   mid   128x128x64, 3 stages, 8 waves: the 128x128 class when a panel is
//         streamed once (tall-skinny), where the deeper ring streams A better;
//   wide  128x128x128, 2 stages, 8 waves: the 128x128 class with reused
//         panels (half as many barriers per K);
//   small 64x64x64, 2 stages, 4 waves: small products.
#define MPG_FAMILY(base, IN, LA, LB)                                                     \
    pipe_entry<PipeCfg<256, 256, 64, 2, 4, 2, LA, LB, IN, 1, 16>>(base + 0),            \
        pipe_entry<PipeCfg<128, 128, 64, 2, 4, 3, LA, LB, IN>>(base + 1),               \
        pipe_entry<PipeCfg<128, 128, 128, 2, 4, 2, LA, LB, IN, 1, 32, 2>>(base + 2),     \
        pipe_entry<PipeCfg<64, 64, 64, 2, 2, 2, LA, LB, IN>>(base + 3)

enum : int { kBig = 0, kMid = 1, kWide = 2, kSmall = 3 };

const Entry kTable[] = {
    direct_entry<kInF16>(0),   // 0      any stride / size / order
    direct_entry<kInBF16>(1),  // 1      BF16 fallback
    scale_entry(2),            // 2      alpha == 0 or K == 0
    MPG_FAMILY(3, kInF16, kRowMajor, kRowMajor),    // 3..6
    MPG_FAMILY(7, kInF16, kColMajor, kRowMajor),    // 7..10
    MPG_FAMILY(11, kInF16, kRowMajor, kColMajor),   // 11..14
    MPG_FAMILY(15, kInF16, kColMajor, kColMajor),   // 15..18
    MPG_FAMILY(19, kInBF16, kRowMajor, kRowMajor),  // 19..22
    MPG_FAMILY(23, kInBF16, kColMajor, kRowMajor),  // 23..26
    MPG_FAMILY(27, kInBF16, kRowMajor, kColMajor),  // 27..30
    MPG_FAMILY(31, kInBF16, kColMajor, kColMajor),  // 31..34
    // small row-major FP16 products with more than one 64-deep K tile: K
    // tiles of 128 on 8 waves of 16x16x32 instructions, 64x64 with a 2-deep
    // ring, or 32x64 with a 3-deep ring when 64x64 tiles would leave more
    // than half of the compute units idle
    pipe_entry<PipeCfg<64, 64, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16>>(35),
    pipe_entry<PipeCfg<32, 64, 128, 2, 4, 3, kRowMajor, kRowMajor, kInF16, 1, 16>>(36),
    // N <= 16 with A row-major, per input format and storage order of B;
    // four k-steps of loads in flight per wave
    narrow_entry<kInF16, kRowMajor, 4>(37),
    narrow_entry<kInF16, kColMajor, 4>(38),
    narrow_entry<kInBF16, kRowMajor, 4>(39),
    narrow_entry<kInBF16, kColMajor, 4>(40),
    // small row-major FP16 products whose 64x64 tiles would leave most of the
    // chip idle and whose B rows hold whole 16-byte vectors: 16x64 tiles on
    // 4 waves, twice the workgroups of 32x64 and fewer bytes copied by each
    pipe_entry<PipeCfg<16, 64, 128, 1, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16>>(41),
#ifdef MPGEMM_CANDIDATES
    // Alternatives the factory does not choose, compiled only into the
    // candidates build for tile sweeps (FP16, A and B row-major).
    pipe_entry<PipeCfg<256, 256, 64, 2, 4, 2>>(42),                   // 32x32x16 on the big tile
    pipe_entry<PipeCfg<256, 256, 32, 2, 2, 4>>(43),                   // 4 waves of 128x128
    pipe_entry<PipeCfg<128, 128, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16, 2>>(44),
    pipe_entry<PipeCfg<128, 128, 128, 2, 2, 2, kRowMajor, kRowMajor, kInF16, 2, 32, 2>>(45),  // 2 k-groups
    pipe_entry<PipeCfg<128, 128, 128, 2, 4, 2>>(46),                  // ascending K order
    pipe_entry<PipeCfg<128, 128, 64, 2, 2, 3>>(47),                   // 4 waves
    pipe_entry<PipeCfg<256, 128, 64, 4, 2, 3>>(48),
    pipe_entry<PipeCfg<128, 128, 64, 2, 4, 3, kRowMajor, kRowMajor, kInF16, 1, 32, 2>>(49),
    pipe_entry<PipeCfg<256, 256, 64, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16, 2>>(50),
    pipe_entry<PipeCfg<64, 64, 128, 2, 2, 3>>(51),                    // 4 waves of 32x32x16
    pipe_entry<PipeCfg<64, 64, 128, 2, 4, 3, kRowMajor, kRowMajor, kInF16, 1, 16>>(52),
    pipe_entry<PipeCfg<32, 64, 128, 2, 2, 3, kRowMajor, kRowMajor, kInF16, 1, 16>>(53),
    narrow_entry<kInF16, kRowMajor, 8>(54),                           // 8 k-steps in flight
    // K orders with more start offsets
    pipe_entry<PipeCfg<128, 128, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 32, 4>>(55),
    pipe_entry<PipeCfg<128, 128, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 32, 8>>(56),
    pipe_entry<PipeCfg<128, 128, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 32, 16>>(57),
    pipe_entry<PipeCfg<64, 64, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16, 64>>(58),
    pipe_entry<PipeCfg<64, 64, 128, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16, 2>>(59),
    pipe_entry<PipeCfg<256, 256, 64, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16, 4>>(60),
    pipe_entry<PipeCfg<256, 256, 64, 2, 4, 2, kRowMajor, kRowMajor, kInF16, 1, 16, 8>>(61),
    pipe_entry<PipeCfg<32, 64, 128, 2, 4, 3, kRowMajor, kRowMajor, kInF16, 1, 16, 64>>(62),
    pipe_entry<PipeCfg<128, 128, 64, 2, 4, 3, kRowMajor, kRowMajor, kInF16, 1, 32, 4>>(63),
    // deeper rings of 64-deep K tiles: more of a streamed A in flight
    pipe_entry<PipeCfg<128, 128, 64, 2, 4, 4>>(64),
    pipe_entry<PipeCfg<128, 128, 64, 2, 4, 5>>(65),
    pipe_entry<PipeCfg<64, 128, 64, 1, 4, 3>>(66),
    pipe_entry<PipeCfg<64, 128, 64, 1, 4, 4>>(67),
    // 16x64 tiles with a 3-deep ring
    pipe_entry<PipeCfg<16, 64, 128, 1, 4, 3, kRowMajor, kRowMajor, kInF16, 1, 16>>(68),
#endif
};
constexpr int kNumEntries = sizeof(kTable) / sizeof(kTable[0]);
constexpr int kDirectIds[2] = {0, 1};  // per input format
constexpr int kScaleId = 2;
// first entry of the family of input format `in` and storage orders (la, lb)
constexpr int family(int in, int la, int lb) { return 3 + 16 * in + 4 * (la + 2 * lb); }
// small row-major FP16 products, K tiles of 128: 64x64, 32x64 and 16x64
constexpr int kSmallDeepKId = 35;
constexpr int kTinyDeepKId = 36;
constexpr int kTiny16Id = 41;
// narrow kernel (N <= 16, A row-major) per input format and storage order of B
constexpr int kNarrowIds[2][2] = {{37, 38}, {39, 40}};
// below this many 16-row workgroups the narrow kernel leaves most compute
// units idle, and split-K over the tile kernels is faster (256x16x65536:
// 74 against 38 us); at or above it the narrow kernel leads (1024x16x16384:
// 21 against 25 us; 4096x16x4096: 7.7 against 16.2)
constexpr int64_t kNarrowMinGroups = 64;

// ---------------------------------------------------------------------------
// Validation and selection (pure host code, no HIP calls)
// ---------------------------------------------------------------------------
struct Problem {
    int64_t M, N, K, lda, ldb, ldc;
    const uint16_t *A;
    const uint16_t *B;
    const float *C;
    float alpha, beta;
    int la, lb;  // storage orders of A and B
    int in_type; // MPGEMM_IN_F16 or MPGEMM_IN_BF16
    const float *bias;  // per-column bias or nullptr
};

int64_t at_least_one(int64_t v) { return v > 1 ? v : 1; }

// Products and sums of caller-supplied sizes (all >= 0 once validated),
// saturated at INT64_MAX instead of overflowing: every size check below
// compares against limits far below it, so a saturated value simply fails
// the check.
int64_t mul_sat(int64_t a, int64_t b)
{
    if (a == 0 || b == 0)
        return 0;
    return a > INT64_MAX / b ? INT64_MAX : a * b;
}

int64_t add_sat(int64_t a, int64_t b) { return a > INT64_MAX - b ? INT64_MAX : a + b; }

int validate(const Problem &p)
{
    if (p.in_type != MPGEMM_IN_F16 && p.in_type != MPGEMM_IN_BF16)
        return MPGEMM_ETYPE;
    if ((p.la != MPGEMM_ROW_MAJOR && p.la != MPGEMM_COL_MAJOR) ||
        (p.lb != MPGEMM_ROW_MAJOR && p.lb != MPGEMM_COL_MAJOR))
        return MPGEMM_ELAYOUT;
    if (p.M < 0 || p.N < 0 || p.K < 0)
        return MPGEMM_EDIM;
    // a stored row holds K values of A (row-major) or M (column-major), N of
    // B (row-major) or K (column-major), N of C
    const int64_t amin = at_least_one(p.la == MPGEMM_COL_MAJOR ? p.M : p.K);
    const int64_t bmin = at_least_one(p.lb == MPGEMM_COL_MAJOR ? p.K : p.N);
    if (p.lda < amin || p.ldb < bmin || p.ldc < at_least_one(p.N))
        return MPGEMM_ELD;
    if (p.M == 0 || p.N == 0)
        return MPGEMM_OK;
    if (p.C == nullptr)
        return MPGEMM_ENULL;
    const bool reads_ab = p.K > 0 && p.alpha != 0.0f;
    if (reads_ab && (p.A == nullptr || p.B == nullptr))
        return MPGEMM_ENULL;
    if ((reinterpret_cast<uintptr_t>(p.C) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(p.bias) & 3u) != 0)
        return MPGEMM_EALIGN;
    if (reads_ab && (((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 1u) != 0))
        return MPGEMM_EALIGN;
    return MPGEMM_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }


// Every valid operand (2-byte aligned, any leading dimension) takes the
// 16-byte copy path: under ROCm, gfx9-family devices run vector memory in
// unaligned mode, where a 16-byte buffer load at any 2-byte aligned address,
// into registers or through the LDS-DMA form, returns exactly the 16 bytes
// there (probed on the device; the parity tests with odd leading dimensions
// and offset pointers run through these paths on every device they run on).

// Can table entry `e` run problem `p`?
bool entry_fits(const Entry &e, const Problem &p)
{
    const mpgemm_config &c = e.cfg;
    const bool trivial = p.M == 0 || p.N == 0;
    const bool scale_only = p.K == 0 || p.alpha == 0.0f;
    if (c.kind == MPGEMM_KIND_SCALE)
        return scale_only || trivial;
    if (c.in_type != p.in_type)
        return false;
    if (c.kind == MPGEMM_KIND_DIRECT)
        return true;
    if (c.layout_a != p.la || c.layout_b != p.lb)
        return false;
    if (trivial || scale_only)
        return true;  // the tiled kernel also handles these; the factory never picks it for them
    if (c.kind == MPGEMM_KIND_NARROW) {
        // 16 stored rows of A, the stored rows of B (K of them row-major, N <= 16
        // column-major) and 16 rows of C within 32-bit buffer offsets
        const int64_t a_span = mul_sat(add_sat(mul_sat(16, p.lda), p.K), 2);
        const int64_t b_span = p.lb == MPGEMM_ROW_MAJOR ? mul_sat(add_sat(mul_sat(p.K, p.ldb), 16), 2)
                                                        : mul_sat(add_sat(mul_sat(16, p.ldb), p.K), 2);
        const int64_t c_span = mul_sat(add_sat(mul_sat(16, p.ldc), 16), 4);
        return p.N <= 16 && a_span < (int64_t)0x7FFFFFF0 && b_span < (int64_t)0x7FFFFFF0 &&
               c_span < (int64_t)0x7FFFFFF0 && cdiv(p.M, 16) <= 0x7FFFFFFF;
    }
    // Per-stage buffer offsets are 32-bit: a stage spans bm (A row-major) or
    // bk (A column-major) stored rows of lda, and bk (B row-major) or bn (B
    // column-major) stored rows of ldb.
    const int64_t a_span = p.la == MPGEMM_ROW_MAJOR ? mul_sat(add_sat(mul_sat(c.bm, p.lda), c.bk), 2)
                                                    : mul_sat(add_sat(mul_sat(c.bk, p.lda), c.bm), 2);
    const int64_t b_span = p.lb == MPGEMM_ROW_MAJOR ? mul_sat(add_sat(mul_sat(c.bk, p.ldb), c.bn), 2)
                                                    : mul_sat(add_sat(mul_sat(c.bn, p.ldb), c.bk), 2);
    if (a_span >= (int64_t)0x7FFFFFF0 || b_span >= (int64_t)0x7FFFFFF0)
        return false;
    // The pipelined kernel's epilogue addresses a wave's C tile with 32-bit
    // buffer offsets as well.
    const int64_t c_span = mul_sat(add_sat(mul_sat(c.bm, p.ldc), c.bn), 4);
    if (c.kind == MPGEMM_KIND_PIPE && c_span >= (int64_t)0x7FFFFFF0)
        return false;
    const int64_t tiles = mul_sat(cdiv(p.M, c.bm), cdiv(p.N, c.bn));
    if (tiles > 0x7FFFFFFF)
        return false;
    return true;
}

int64_t grid_for(const mpgemm_config &c, const Problem &p)
{
    switch (c.kind) {
    case MPGEMM_KIND_PIPE:
        return mul_sat(cdiv(p.M, c.bm), cdiv(p.N, c.bn));
    case MPGEMM_KIND_DIRECT:
        return mul_sat(cdiv(p.M, 64), cdiv(p.N, 64));
    case MPGEMM_KIND_NARROW:
        return cdiv(p.M, 16);
    case MPGEMM_KIND_SCALE:
        return 0;
    default:
        return 0;
    }
}

// The factory.  The tile by rounds of workgroups over the compute units;
// smaller tiles when the product is small.  Returns a table id, or -1 for
// "nothing to do".
// `small_deep_k` = false keeps 64-deep K tiles for small products (split-K
// counts its pieces in K tiles).
int select(const Problem &p, bool small_deep_k = true, bool allow_narrow = true)
{
    if (p.M == 0 || p.N == 0)
        return -1;
    if (p.K == 0 || p.alpha == 0.0f)
        return kScaleId;
    // At most 16 columns with A row-major: a stream over A, taken by the
    // narrow kernel (16 rows per workgroup, K split over its waves).
    if (allow_narrow && p.N <= 16 && p.la == MPGEMM_ROW_MAJOR) {
        const int nid = kNarrowIds[p.in_type][p.lb];
        if (entry_fits(kTable[nid], p))
            return nid;
    }
    // 256x256 for large products (by rounds, below).
    // Else 128x128 if that makes at least half a wave of workgroups.
    // Else 64x64.
    const int fam = family(p.in_type, p.la, p.lb);
    // Small row-major FP16 products with more than one 64-deep K tile have
    // K tiles of 128 and the 16x16x32 instruction (half as many barriers
    // per K).
    const bool deep_k = small_deep_k && p.in_type == MPGEMM_IN_F16 && p.la == MPGEMM_ROW_MAJOR &&
                        p.lb == MPGEMM_ROW_MAJOR && p.K > 64;
    const int64_t tiles64 = mul_sat(cdiv(p.M, 64), cdiv(p.N, 64));
    int order[6];
    int n = 0;
    // 256x256 or 128x128 tiles, by the rounds of workgroups each puts on
    // the compute units (one workgroup per unit): a 256x256 tile takes about
    // three times as long as a 128x128 one (4096^3: 133.8 us for one round
    // of 256 against 44.3 per round of 128x128 tiles), and a round that
    // leaves units idle takes about as long as a full one.  So the big tile
    // wins when 3 * its rounds <= the 128x128 rounds (3072x2816x4096: 106.4
    // against 123.4 us with 132 big tiles; 4352x4096x4096: 230.6 against
    // 209.1 with 272, two rounds, for 5 rounds of 128x128; the same for
    // both input formats and every storage order).  A product with one
    // 128-row or 128-column band never takes it: its 256x256 tiles would be
    // at least half empty (65536x128x4096 159.7 against 130.2 us).
    const bool rr16 = p.in_type == MPGEMM_IN_F16 && p.la == MPGEMM_ROW_MAJOR && p.lb == MPGEMM_ROW_MAJOR;
    const int64_t tm128 = cdiv(p.M, 128), tn128 = cdiv(p.N, 128);
    const int64_t tiles256 = mul_sat(cdiv(p.M, 256), cdiv(p.N, 256));
    const int64_t rounds256 = cdiv(tiles256, kNumCu);
    const int64_t rounds128 = cdiv(mul_sat(tm128, tn128), kNumCu);
    // With A row-major and B column-major (both K-contiguous, every operand
    // read by ds_read_b128) the big tile is relatively cheaper: it wins at
    // 2.5 times its rounds (1504x12052x2229, two rounds against five: 150.3
    // against 171.5 us; 7198x2381x2219 148.5 against 168.4; 1018x16708x510
    // 49.5 against 53.2; 4352x4096x4096 201.0 against 197.7 the one loss).
    const bool big_by_rounds = (p.la == MPGEMM_ROW_MAJOR && p.lb == MPGEMM_COL_MAJOR)
                                   ? mul_sat(5, rounds256) <= mul_sat(2, rounds128)
                                   : mul_sat(3, rounds256) <= rounds128;
    // Short K (at most 256) over at least two 64x64 tiles per compute unit:
    // writing C is much of the work, and the 64x64x64 tiles on 4 waves,
    // several workgroups per unit, overlap one tile's stores with another's
    // loads.  They win unless the 256x256 tiles come to nearly a full round
    // (at least 240 of them: 4096^2 x 64 14.6 against 16.6 us, 1456x10608x128
    // 16.8 against 18.5) or the 128x128 class has whole 128-deep K tiles
    // (2048^2 x 128 6.48 against 6.59): 3328^2 x 128 12.8 against 14.4 us
    // for 169 big tiles, 6144x2048x192 16.2 against 16.5, 2048^2 x 192 7.0
    // against 7.9, 2048x1024x192 5.3 against 6.2, 5907x1622x137 18.9
    // against 26.3.
    if (p.K <= 256 && tiles64 >= 2 * kNumCu) {
        if (big_by_rounds && tiles256 >= 240)
            order[n++] = fam + kBig;
        else if (!big_by_rounds && p.K % 128 == 0)
            order[n++] = fam + kWide;
        order[n++] = fam + kSmall;
        order[n++] = fam + kMid;
    } else if (big_by_rounds) {
        order[n++] = fam + kBig;
        order[n++] = fam + kMid;
    } else if (mul_sat(cdiv(p.M, 128), cdiv(p.N, 128)) >= kNumCu / 2 &&
               !(deep_k && tiles64 <= 2 * kNumCu)) {
        // (Half a wave of 128x128 tiles whose 64x64 tiles come to at most
        // two per compute unit runs faster as 64x64 tiles on every unit:
        // 1024x2048x2048 17.7 against 22.0 us, graph-replayed.)
        // 128x128 tiles take K steps of 128 (half as many barriers) when
        // both panels are reused across tiles, by graph-replayed sweeps of
        // the two shapes (row-major FP16; the BF16 and column-major forms
        // follow the same pattern): at least two tile rows and two tile
        // columns (16384x256x4096 49.3 against 55.4 us, 8192x384x1024 13.0
        // against 14.7, 256x16384x4096 48.6 against 55.5), except two tile
        // columns from K = 8192 (32768x256x8192 196.5 against 225.4); one
        // tile column, where A is streamed once, only up to K = 1024
        // (32768x128x1024 16.9 against 17.6; x4096 62.7 against 58.5 for
        // the deeper 64-wide ring); one tile row, where B is streamed once,
        // up to K = 2048 (128x32768x2048 28.3 against 29.7; 128x65536x4096
        // 143.3 against 122.1).
        const bool wide = (tm128 >= 2 && tn128 >= 2 && !(tn128 == 2 && p.K >= 8192)) ||
                          (tn128 == 1 && p.K <= 1024) || (tm128 == 1 && p.K <= 2048);
        // Row-major FP16 whose B rows are not 16-byte aligned, with a second
        // round of at most 64 128x128 tiles: the 64x64x128 tiles (two
        // workgroups per unit) balance the tail better (2049^2 x 2048 57.0
        // against 60.6 us, 2048x2049x2048 57.3 against 64.5, 2100^2 x 2048
        // 57.9 against 64.3, 1744x2439x2048 59.4 against 63.8; with aligned
        // B rows the 128x128 tiles keep the lead: 2049x2048x2048 42.4
        // against 44.2).
        const int64_t tail128 = mul_sat(tm128, tn128) - kNumCu;
        if (small_deep_k && rr16 && p.ldb % 8 != 0 && rounds128 == 2 && tail128 <= 64)
            order[n++] = kSmallDeepKId;
        if (wide)
            order[n++] = fam + kWide;
        order[n++] = fam + kMid;
    } else if (deep_k) {
        // Fewer 64x64 tiles than compute units (times graph-replayed):
        // * 16x64 tiles on 4 waves while they come to at most one per unit
        //   and K is moderate (256^3: 3.34 against 3.66 us for 32x64 and
        //   3.94 for 64x64; 512x512x2048 9.98 against 10.56 and 11.32), and
        //   N a multiple of 8 -- otherwise the last column of tiles fills
        //   partial B vectors through registers on every K tile, which 8
        //   waves share better (200x300x400: 6.7 against 8.1 us for 32x64);
        // * else 32x64 tiles on 8 waves with a 3-deep ring while they come
        //   to at most one per unit (512x768x1024 6.85 against 7.22 for
        //   16x64 and 7.29 for 64x64) or K is long (the deeper ring keeps
        //   pace where the 2-deep ones fall behind: 512x512x8192 33.9
        //   against 43.5 for 16x64 and 46.7 for 64x64; 768x768x8192 45.3
        //   against 47.7 for 64x64);
        // * else 64x64 on 8 waves (ragged 1000x800x617: 7.1 against 7.3 us
        //   for 4 waves).
        if (tiles64 < kNumCu) {
            const int64_t tiles16 = mul_sat(cdiv(p.M, 16), cdiv(p.N, 64));
            const int64_t tiles32 = mul_sat(cdiv(p.M, 32), cdiv(p.N, 64));
            if (p.N % 8 == 0 && ((tiles16 <= kNumCu && p.K <= 2048) || (tiles16 <= kNumCu / 2 && p.K <= 4096)))
                order[n++] = kTiny16Id;
            if (tiles32 <= kNumCu || p.K >= 4096)
                order[n++] = kTinyDeepKId;
        }
        order[n++] = kSmallDeepKId;
    }
    order[n++] = fam + kSmall;
    for (int i = 0; i < n; ++i)
        if (entry_fits(kTable[order[i]], p))
            return order[i];
    // Leading dimensions so large that the preferred tiles' stages overflow
    // 32-bit offsets: any other tiled entry whose stages fit (the smallest
    // tiles first) before the 64-bit direct kernel.
    const int rest[] = {rr16 ? kTiny16Id : -1, rr16 ? kTinyDeepKId : -1, rr16 ? kSmallDeepKId : -1,
                        fam + kMid, fam + kWide, fam + kBig};
    for (int id : rest)
        if (id >= 0 && entry_fits(kTable[id], p))
            return id;
    return kDirectIds[p.in_type];
}

// A one-column B stored row-major with ldb == 1 is K consecutive values: the
// same bytes as a column-major B with ldb == K.  When the narrow kernel takes
// the product, the factory reads B in that form: the narrow kernel's
// column-major loads are K-contiguous and 16-byte aligned (4096x1x4096: 6.8
// against 9.7 us, bitwise the same results).  Other kernels keep the order
// given (a column-major stage spans ldb = K per column, which can push a
// huge K past the tiled kernels' 32-bit offsets).  Applied after validation,
// so the caller's arguments are checked as given.
Problem canonical(Problem p)
{
    if (p.N != 1 || p.lb != MPGEMM_ROW_MAJOR || p.ldb != 1)
        return p;
    Problem q = p;
    q.lb = MPGEMM_COL_MAJOR;
    q.ldb = at_least_one(p.K);
    const int id = select(q);
    return id >= 0 && kTable[id].cfg.kind == MPGEMM_KIND_NARROW ? q : p;
}

// Cache policy of the pipelined kernel's C stores, by graph-replayed A/B of
// the two policies.  Non-temporal stores keep C from evicting the operand
// panels and win for 128x128 and smaller tiles, which have that variant
// only (2048^3 24.5 against 25.7 us, 32768x128x4096 52.9 against 57.7,
// 16384x256x1024 14.2 against 15.8; rows that start mid-line make no
// difference there: 2049^2 x 2048 59.0 against 58.9).  256x256 tiles write
// up to 64 MiB of C per round at once, which plain stores let the caches
// absorb from about 190 tiles on (6144x2048x1024, 192 tiles, 32.8 against
// 33.5 us; 3584x4096x1024, 224, 35.2 against 36.3; 8192x8192x512 103.9
// against 117.5; 4096^3 113.0 against 116.1); with fewer tiles (up to 169
// measured: 3328^2 x 512 21.1 against 21.4, 2560^2 x 512 18.5 against
// 20.6) or more than one round at long K (8192^3 855 against 881,
// 8192x8192x2048 262.0 against 265.0) non-temporal stores win.  Rows that
// start mid-line (ldc not a multiple of 32 floats, or C not 128-byte
// aligned) take plain stores: there non-temporal partial lines cost up to
// 2.5x (1457x10609x128: 16.8 against 42.1 us).
bool nt_stores(const mpgemm_config &c, const Problem &p)
{
    if (c.kind != MPGEMM_KIND_PIPE || c.bm < 256)
        return true;
    const bool aligned = p.ldc % 32 == 0 && (reinterpret_cast<uintptr_t>(p.C) & 127) == 0;
    const int64_t tiles = mul_sat(cdiv(p.M, c.bm), cdiv(p.N, c.bn));
    return aligned && (tiles <= 176 || (tiles > kNumCu && p.K >= 2048));
}

int fill_config(int id, const Problem &p, mpgemm_config *out)
{
    if (id < 0) {
        mpgemm_config c{};
        c.id = -1;
        c.kind = MPGEMM_KIND_NONE;
        c.layout_a = p.la;
        c.layout_b = p.lb;
        c.in_type = p.in_type;
        c.k_groups = 1;
        *out = c;
        return MPGEMM_OK;
    }
    *out = kTable[id].cfg;
    out->grid = grid_for(out[0], p);
    if (out->kind == MPGEMM_KIND_PIPE)
        out->c_stores = nt_stores(*out, p) ? 1 : 0;
    out->layout_a = p.la;
    out->layout_b = p.lb;
    out->in_type = p.in_type;
    return MPGEMM_OK;
}


int run(int id, const Problem &p, void *stream)
{
    if (id < 0)
        return MPGEMM_OK;
    const Entry &e = kTable[id];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (e.cfg.kind == MPGEMM_KIND_SCALE || p.K == 0 || p.alpha == 0.0f) {
        if (p.M == 0 || p.N == 0)
            return MPGEMM_OK;
        const int64_t gx = cdiv(p.N, 256) < 64 ? cdiv(p.N, 256) : 64;
        const int64_t gy = p.M < 65535 ? p.M : 65535;
        (void)hipGetLastError();  // not an earlier call's error
        hipLaunchKernelGGL(mpg::scale_c, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s,
                           const_cast<float *>(p.C), p.M, p.N, p.ldc, p.beta, p.bias);
        return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
    }
    GemmArgs a;
    a.A = p.A;
    a.B = p.B;
    a.C = const_cast<float *>(p.C);
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.a_i = p.la == MPGEMM_COL_MAJOR ? 1 : p.lda;
    a.a_k = p.la == MPGEMM_COL_MAJOR ? p.lda : 1;
    a.b_k = p.lb == MPGEMM_COL_MAJOR ? 1 : p.ldb;
    a.b_j = p.lb == MPGEMM_COL_MAJOR ? p.ldb : 1;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.bias = p.bias;
    a.splits = 1;
    a.k_split = 0;
    a.ws = nullptr;
    const int64_t grid = grid_for(e.cfg, p);
    if (e.cfg.kind == MPGEMM_KIND_DIRECT) {
        a.tiles_m = (int32_t)cdiv(p.M, 64);
        a.tiles_n = (int32_t)cdiv(p.N, 64);
    } else if (e.cfg.kind == MPGEMM_KIND_NARROW) {
        a.tiles_m = (int32_t)cdiv(p.M, 16);
        a.tiles_n = 1;
    } else {
        a.tiles_m = (int32_t)cdiv(p.M, e.cfg.bm);
        a.tiles_n = (int32_t)cdiv(p.N, e.cfg.bn);
    }
    a.group_m = 8;
    if (grid <= 0 || grid > 0x7FFFFFFF)
        return MPGEMM_ECONFIG;
    // A launch error from an earlier, unrelated call must not be reported
    // as this call's failure.
    (void)hipGetLastError();
    const launch_fn launch = nt_stores(e.cfg, p) ? e.launch : e.launch_plain;
    const hipError_t err = launch(a, dim3((unsigned)grid), s);
    return err == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}

// ---------------------------------------------------------------------------
// Split-K for grids that leave compute units idle
// ---------------------------------------------------------------------------
struct SplitPlan {
    int id;           // table entry of the tile kernel
    int splits;       // K ranges (1: no split)
    int64_t k_split;  // elements of K per range, a multiple of the entry's bk
    int64_t ws_bytes; // workspace the partial products need
};

// `requested` 0: automatic (split only a grid under one wave of resident
// workgroups with K >= 4096, into ranges of about 1024 K, at most about 4
// workgroups per compute unit and at most 32 ranges); otherwise that many
// ranges, at most one per K tile.  Empty ranges are never planned.
SplitPlan plan_split(const Problem &p, int requested)
{
    // an unsplit plan keeps the factory's own choice
    SplitPlan sp{select(p), 1, 0, 0};
    if (sp.id < 0 || p.K == 0 || p.alpha == 0.0f)
        return sp;
    // The narrow kernel splits K inside its workgroups: the automatic plan
    // keeps it unless its grid has few 16-row workgroups, where split-K over
    // the tile kernels is faster; a requested piece count splits a tile
    // kernel.  Pieces are whole K tiles: a split takes the 64-deep form of
    // the small tile.
    const bool narrow = kTable[sp.id].cfg.kind == MPGEMM_KIND_NARROW;
    if (narrow && requested == 0 && cdiv(p.M, 16) >= kNarrowMinGroups)
        return sp;
    int id = narrow ? select(p, true, false) : sp.id;
    if (id == kSmallDeepKId || id == kTinyDeepKId || id == kTiny16Id)
        id = select(p, false, false);
    const mpgemm_config &c = kTable[id].cfg;
    if (c.kind != MPGEMM_KIND_PIPE)
        return sp;
    const int64_t tiles = grid_for(c, p);
    const int64_t ktiles = cdiv(p.K, c.bk);
    int64_t s;
    if (requested == 0) {
        // Only grids under one wave of resident workgroups (the config's
        // LDS allows `occ` per compute unit), only K of at least 4096, and
        // pieces of about 1024 K, at most about 4 workgroups per unit and at
        // most 32 pieces.  By graph-replayed sweeps of forced piece counts:
        // 256x256x8192 8 pieces 16.0 us (32 pieces 22.7, unsplit 33.5),
        // 256x256x65536 32 pieces 45.2, 2048x256x8192 8 pieces 26.8
        // (unsplit 36.1), 1024x1024x8192 4 pieces 41.5 (unsplit 48.0);
        // shorter K stays whole (512x512x2048 unsplit 10.3 against 13.5 for
        // 2 pieces and 14.1 for 8).  A grid of at most 64 tiles takes at
        // least 8 pieces (pieces of 512 K and more): 256x96x5000 12.5 us in
        // 8 against 15.0 in 4, 256x256x4096 12.4 against 13.5, 512x48x4096
        // 11.8 against 13.3.  A larger one takes at least 6 while that keeps
        // it within 4 workgroups per unit: 640x640x4096 17.4 in 6 against
        // 19.2 in 4, 1536x256x4096 17.5 against 19.3 (1024x1024x4096, 256
        // tiles, keeps 4: 26.9 against 31.1 in 6).
        const int64_t occ = c.lds_bytes > 0 ? (160 * 1024) / c.lds_bytes : 1;
        const int64_t resident = kNumCu * (occ < 1 ? 1 : occ > 4 ? 4 : occ);
        if (tiles >= resident || p.K < 4096)
            s = 1;
        else {
            s = p.K / 1024;
            const int64_t floor_s = tiles <= 64 ? 8 : 6;
            if (s < floor_s && tiles * floor_s <= 4 * kNumCu)
                s = floor_s;
            const int64_t cap = cdiv(4 * kNumCu, tiles);
            if (s > cap)
                s = cap;
            if (s > 32)
                s = 32;
        }
    } else {
        s = requested < ktiles ? requested : ktiles;
    }
    if (s <= 1)
        return sp;
    const int64_t k_split = mul_sat(cdiv(ktiles, s), c.bk);
    const int64_t pieces = cdiv(p.K, k_split);
    // the workspace holds one M x N FP32 product per piece
    const int64_t ws_bytes = mul_sat(mul_sat(mul_sat(pieces, p.M), p.N), 4);
    if (pieces <= 1 || mul_sat(tiles, pieces) > 0x7FFFFFFF || ws_bytes == INT64_MAX)
        return sp;
    sp.id = id;
    sp.k_split = k_split;
    sp.splits = (int)pieces;
    sp.ws_bytes = ws_bytes;
    return sp;
}

int run_split(const SplitPlan &sp, const Problem &p, float *ws, void *stream)
{
    const Entry &e = kTable[sp.id];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    GemmArgs a{};
    a.A = p.A;
    a.B = p.B;
    a.C = const_cast<float *>(p.C);
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.bias = p.bias;
    a.tiles_m = (int32_t)cdiv(p.M, e.cfg.bm);
    a.tiles_n = (int32_t)cdiv(p.N, e.cfg.bn);
    a.group_m = 8;
    a.splits = sp.splits;
    a.k_split = sp.k_split;
    a.ws = ws;

    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * sp.splits;
    (void)hipGetLastError();
    hipError_t err = e.launch(a, dim3((unsigned)grid), s);
    if (err != hipSuccess)
        return MPGEMM_ELAUNCH;
    const int64_t gx = cdiv(p.N, 256) < 64 ? cdiv(p.N, 256) : 64;
    const int64_t gy = p.M < 65535 ? p.M : 65535;
    hipLaunchKernelGGL(mpg::splitk_reduce, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s,
                       const_cast<float *>(p.C), p.M, p.N, p.ldc, ws, sp.splits, p.alpha, p.beta,
                       p.bias);
    return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}

Problem make_problem(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                     const uint16_t *B, int64_t ldb, const float *C, int64_t ldc,
                     float alpha, float beta, int la = MPGEMM_ROW_MAJOR, int lb = MPGEMM_ROW_MAJOR,
                     int in_type = MPGEMM_IN_F16, const float *bias = nullptr)
{
    return Problem{M, N, K, lda, ldb, ldc, A, B, C, alpha, beta, la, lb, in_type, bias};
}

int gemm_layout(int in_type, int la, int lb, int64_t M, int64_t N, int64_t K, const uint16_t *A,
                int64_t lda, const uint16_t *B, int64_t ldb, float *C, int64_t ldc, float alpha,
                float beta, void *stream, const float *bias = nullptr)
{
    const Problem given = make_problem(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, la, lb, in_type,
                                   bias);
    const int rc = validate(given);
    if (rc != MPGEMM_OK)
        return rc;
    const Problem p = canonical(given);
    return run(select(p), p, stream);
}

int query_layout(int in_type, int la, int lb, int64_t M, int64_t N, int64_t K, const uint16_t *A,
                 int64_t lda, const uint16_t *B, int64_t ldb, const float *C, int64_t ldc,
                 float alpha, float beta, mpgemm_config *out)
{
    if (out == nullptr)
        return MPGEMM_ENULL;
    const Problem given = make_problem(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, la, lb, in_type);
    const int rc = validate(given);
    if (rc != MPGEMM_OK)
        return rc;
    const Problem p = canonical(given);
    return fill_config(select(p), p, out);
}

int with_config_layout(int in_type, int config_id, int la, int lb, int64_t M, int64_t N,
                       int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       float *C, int64_t ldc, float alpha, float beta, void *stream,
                       const float *bias = nullptr)
{
    if (config_id < 0 || config_id >= kNumEntries)
        return MPGEMM_ECONFIG;
    const Problem p = make_problem(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, la, lb, in_type,
                                   bias);
    const int rc = validate(p);
    if (rc != MPGEMM_OK)
        return rc;
    if (!entry_fits(kTable[config_id], p))
        return MPGEMM_ECONFIG;
    if (p.M == 0 || p.N == 0)
        return MPGEMM_OK;
    return run(config_id, p, stream);
}

// ---------------------------------------------------------------------------
// Static split-K scratch for callers that cannot allocate
// ---------------------------------------------------------------------------
// The array itself (`scratch`, at file scope below the namespace) exists
// once per device: the code object is loaded on every device the library
// runs on, and each holds its own copy until the process ends.  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr int64_t kScratchBytes = MPGEMM_STATIC_SCRATCH_BYTES;
int scratch_address(void **out);

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address into *out (looked up on its first
// use on that device).  MPGEMM_ELAUNCH if the runtime refuses.
int scratch_for_current_device(float **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MPGEMM_ELAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (scratch_address(&ptr) != MPGEMM_OK || ptr == nullptr)
            return MPGEMM_ELAUNCH;
        g_scratch_ptr[dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return MPGEMM_OK;
}

}  // namespace

// Partial products of mpgemm_gemm_splitk_static (file scope, one per device).
static __device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {
// The current device's address of `scratch`.
int scratch_address(void **out)
{
    return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)) == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}
}  // namespace

extern "C" {

int mpgemm_f16f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                  const uint16_t *B, int64_t ldb, float *C, int64_t ldc, float alpha,
                  float beta, void *stream)
{
    return gemm_layout(MPGEMM_IN_F16, MPGEMM_ROW_MAJOR, MPGEMM_ROW_MAJOR, M, N, K, A, lda, B, ldb,
                       C, ldc, alpha, beta, stream);
}

int mpgemm_f16f32_query(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb, const float *C, int64_t ldc,
                        float alpha, float beta, mpgemm_config *out)
{
    return query_layout(MPGEMM_IN_F16, MPGEMM_ROW_MAJOR, MPGEMM_ROW_MAJOR, M, N, K, A, lda, B, ldb,
                        C, ldc, alpha, beta, out);
}

int mpgemm_f16f32_with_config(int config_id, int64_t M, int64_t N, int64_t K,
                              const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                              float *C, int64_t ldc, float alpha, float beta, void *stream)
{
    return with_config_layout(MPGEMM_IN_F16, config_id, MPGEMM_ROW_MAJOR, MPGEMM_ROW_MAJOR, M, N, K,
                              A, lda, B, ldb, C, ldc, alpha, beta, stream);
}

int mpgemm_f16f32_layout(int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                         float *C, int64_t ldc, float alpha, float beta, void *stream)
{
    return gemm_layout(MPGEMM_IN_F16, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                       beta, stream);
}

int mpgemm_f16f32_layout_query(int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                               const float *C, int64_t ldc, float alpha, float beta,
                               mpgemm_config *out)
{
    return query_layout(MPGEMM_IN_F16, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                        beta, out);
}

int mpgemm_f16f32_layout_with_config(int config_id, int layout_a, int layout_b, int64_t M,
                                     int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                                     const uint16_t *B, int64_t ldb, float *C, int64_t ldc,
                                     float alpha, float beta, void *stream)
{
    return with_config_layout(MPGEMM_IN_F16, config_id, layout_a, layout_b, M, N, K, A, lda, B, ldb,
                              C, ldc, alpha, beta, stream);
}

int mpgemm_bf16f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb, float *C, int64_t ldc, float alpha,
                   float beta, void *stream)
{
    return gemm_layout(MPGEMM_IN_BF16, MPGEMM_ROW_MAJOR, MPGEMM_ROW_MAJOR, M, N, K, A, lda, B, ldb,
                       C, ldc, alpha, beta, stream);
}

int mpgemm_bf16f32_layout(int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          float *C, int64_t ldc, float alpha, float beta, void *stream)
{
    return gemm_layout(MPGEMM_IN_BF16, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                       beta, stream);
}

int mpgemm_bf16f32_layout_query(int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                                const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                                const float *C, int64_t ldc, float alpha, float beta,
                                mpgemm_config *out)
{
    return query_layout(MPGEMM_IN_BF16, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                        beta, out);
}

int mpgemm_bf16f32_layout_with_config(int config_id, int layout_a, int layout_b, int64_t M,
                                      int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                                      const uint16_t *B, int64_t ldb, float *C, int64_t ldc,
                                      float alpha, float beta, void *stream)
{
    return with_config_layout(MPGEMM_IN_BF16, config_id, layout_a, layout_b, M, N, K, A, lda, B,
                              ldb, C, ldc, alpha, beta, stream);
}

int mpgemm_gemm_ex(int in_type, int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float *C,
                   int64_t ldc, float alpha, float beta, const float *bias, void *stream)
{
    return gemm_layout(in_type, layout_a, layout_b, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                       stream, bias);
}

int mpgemm_gemm_ex_with_config(int config_id, int in_type, int layout_a, int layout_b, int64_t M,
                               int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb, float *C, int64_t ldc, float alpha,
                               float beta, const float *bias, void *stream)
{
    return with_config_layout(in_type, config_id, layout_a, layout_b, M, N, K, A, lda, B, ldb, C,
                              ldc, alpha, beta, stream, bias);
}

int mpgemm_splitk_plan(int in_type, int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       int splits_requested, int32_t *splits, int64_t *workspace_bytes,
                       int32_t *config_id)
{
    if (splits_requested < 0)
        return MPGEMM_ESPLIT;
    // C is not touched by planning: any aligned stand-in passes validation
    static const float c_stand_in = 0.0f;
    const Problem given = make_problem(M, N, K, A, lda, B, ldb, &c_stand_in, N > 1 ? N : 1, 1.0f,
                                   0.0f, layout_a, layout_b, in_type);
    const int rc = validate(given);
    if (rc != MPGEMM_OK)
        return rc;
    const Problem p = canonical(given);
    const SplitPlan sp = plan_split(p, splits_requested);
    if (splits)
        *splits = sp.splits;
    if (workspace_bytes)
        *workspace_bytes = sp.ws_bytes;
    if (config_id)
        *config_id = sp.id;
    return MPGEMM_OK;
}

int mpgemm_gemm_splitk(int in_type, int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float *C,
                       int64_t ldc, float alpha, float beta, const float *bias,
                       int splits_requested, float *workspace, int64_t workspace_bytes,
                       void *stream)
{
    if (splits_requested < 0)
        return MPGEMM_ESPLIT;
    const Problem given = make_problem(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, layout_a,
                                   layout_b, in_type, bias);
    const int rc = validate(given);
    if (rc != MPGEMM_OK)
        return rc;
    const Problem p = canonical(given);
    const SplitPlan sp = plan_split(p, splits_requested);
    if (sp.splits <= 1)
        return run(sp.id, p, stream);
    if (workspace == nullptr)
        return MPGEMM_ENULL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0)
        return MPGEMM_EALIGN;
    if (workspace_bytes < sp.ws_bytes)
        return MPGEMM_EWORKSPACE;
    return run_split(sp, p, workspace, stream);
}

int mpgemm_gemm_splitk_static(int in_type, int layout_a, int layout_b, int64_t M, int64_t N, int64_t K,
                              const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float *C,
                              int64_t ldc, float alpha, float beta, const float *bias,
                              int splits_requested, void *stream)
{
    if (splits_requested < 0)
        return MPGEMM_ESPLIT;
    const Problem given = make_problem(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, layout_a,
                                   layout_b, in_type, bias);
    const int rc = validate(given);
    if (rc != MPGEMM_OK)
        return rc;
    const Problem p = canonical(given);
    SplitPlan sp = plan_split(p, splits_requested);
    if (splits_requested == 0 && sp.splits > 1 && sp.ws_bytes > kScratchBytes) {
        // an automatic plan larger than the scratch: as many pieces as fit
        // (the unsplit product when fewer than two do)
        const int64_t fit = kScratchBytes / mul_sat(mul_sat(p.M, p.N), 4);
        sp = fit >= 2 ? plan_split(p, (int)(fit < 32 ? fit : 32)) : SplitPlan{select(p), 1, 0, 0};
    }
    if (sp.splits <= 1)
        return run(sp.id, p, stream);
    if (sp.ws_bytes > kScratchBytes)
        return MPGEMM_ESCRATCH;
    float *ws = nullptr;
    const int src = scratch_for_current_device(&ws);
    if (src != MPGEMM_OK)
        return src;
    return run_split(sp, p, ws, stream);
}

int mpgemm_num_configs(void) { return kNumEntries; }

int mpgemm_config_info(int config_id, mpgemm_config *out)
{
    if (config_id < 0 || config_id >= kNumEntries)
        return MPGEMM_ECONFIG;
    if (out == nullptr)
        return MPGEMM_ENULL;
    *out = kTable[config_id].cfg;
    return MPGEMM_OK;
}

const char *mpgemm_strerror(int code)
{
    switch (code) {
    case MPGEMM_OK:
        return "success";
    case MPGEMM_EDIM:
        return "a dimension is negative";
    case MPGEMM_ELD:
        return "a leading dimension is smaller than its row length";
    case MPGEMM_ENULL:
        return "a required pointer is NULL";
    case MPGEMM_ELAUNCH:
        return "the HIP kernel launch failed";
    case MPGEMM_ECONFIG:
        return "unknown config, or the config cannot run these arguments";
    case MPGEMM_EALIGN:
        return "A/B are not 2-byte aligned or C is not 4-byte aligned";
    case MPGEMM_ELAYOUT:
        return "a layout is neither MPGEMM_ROW_MAJOR nor MPGEMM_COL_MAJOR";
    case MPGEMM_ETYPE:
        return "the input type is neither MPGEMM_IN_F16 nor MPGEMM_IN_BF16";
    case MPGEMM_EWORKSPACE:
        return "the split-K workspace is smaller than mpgemm_splitk_plan reports";
    case MPGEMM_ESPLIT:
        return "a negative split count was requested";
    case MPGEMM_ESCRATCH:
        return "the split-K plan needs more than the static scratch (MPGEMM_STATIC_SCRATCH_BYTES)";
    default:
        return "unknown error code";
    }
}

const char *mpgemm_version(void) { return "mpgemm 0.8.0 gfx950"; }

#ifdef MPGEMM_TIMELINE
// Timeline build only: host access to the per-workgroup stamps the
// pipelined kernel leaves in mpg::g_timeline.
int64_t mpgemm_timeline_entries(void) { return (int64_t)mpg::kTimelineWgs * mpg::kTimelineSlots; }

int mpgemm_timeline_read(uint64_t *out, int64_t entries)
{
    if (out == nullptr)
        return MPGEMM_ENULL;
    if (entries < 0 || entries > mpgemm_timeline_entries())
        return MPGEMM_EDIM;
    if (entries == 0)
        return MPGEMM_OK;
    if (hipDeviceSynchronize() != hipSuccess)
        return MPGEMM_ELAUNCH;
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(mpg::g_timeline), (size_t)entries * sizeof(uint64_t), 0,
                               hipMemcpyDeviceToHost) == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}

int mpgemm_timeline_clear(void)
{
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(mpg::g_timeline)) != hipSuccess || p == nullptr)
        return MPGEMM_ELAUNCH;
    if (hipMemset(p, 0, (size_t)mpgemm_timeline_entries() * sizeof(uint64_t)) != hipSuccess)
        return MPGEMM_ELAUNCH;
    return hipDeviceSynchronize() == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}
#endif

}  // extern "C"
