// probes.hip -- diagnostics for the gfx950 GEMM (libmpgemm_probes.so; C ABI
// in include/mpgemm_probes.h): the matrix-instruction lane layout, sustained
// matrix-core throughput, and the L2 fill rate per XCD.  They share the
// GEMM's device helpers (instruction wrappers, buffer descriptors, the
// direct-to-LDS copy) but none of its kernels, and are not linked into the
// product library.
#include "mpgemm.h"
#include "mpgemm_probes.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace mpg {

// One wave.  A[i][0] = i, A[i][1] = 1, B[0][j] = 1, B[1][j] = S*j, the rest
// zero, so D[i][j] = i + S*j; each lane writes its accumulators in order.
__global__ void __launch_bounds__(64)
probe_mfma(float *out, int shape)
{
    const int l = threadIdx.x;
    half8 a = half8{0}, b = half8{0};
    if (shape == 32) {
        if (l < 32) {  // k = 0..7 held by lanes 0..31
            a[0] = (_Float16)(float)(l & 31);
            a[1] = (_Float16)1.0f;
            b[0] = (_Float16)1.0f;
            b[1] = (_Float16)(float)(32 * (l & 31));
        }
        floatx16 d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, floatx16{0}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v)
            out[l * 16 + v] = d[v];
    } else {
        if (l < 16) {  // k = 0..7 held by lanes 0..15
            a[0] = (_Float16)(float)(l & 15);
            a[1] = (_Float16)1.0f;
            b[0] = (_Float16)1.0f;
            b[1] = (_Float16)(float)(16 * (l & 15));
        }
        floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, floatx4{0}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[l * 4 + v] = d[v];
    }
}

// Matrix-core throughput probe.  Every wave loads four operand pairs once
// (lane l: A values ops[64*(16*q + l)/8 ...], see below) and then issues
// `iters` rounds of MFMA_N independent matrix instructions, rotating through
// the four pairs so consecutive instructions see different operand bits, as
// in the GEMM's inner loop; nothing touches memory inside the loop.  Each
// lane writes the sum of its accumulators to out[global thread id], so the
// work is kept.  A diagnostic of the clock and power the matrix cores settle
// at under sustained load for given operand values.
// ops: 4 pairs x 64 lanes x 16 values (8 for A, then 8 for B) = 4096 values.
template <int IN, int MI>
__global__ void __launch_bounds__(512)
probe_mfma_rate(const uint16_t *ops, int64_t iters, float *out)
{
    const int lane = threadIdx.x & 63;
    half8 a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[q][e] = __builtin_bit_cast(_Float16, ops[(q * 64 + lane) * 16 + e]);
            b[q][e] = __builtin_bit_cast(_Float16, ops[(q * 64 + lane) * 16 + 8 + e]);
        }
    // 128 accumulator registers per lane, like the GEMM's wave tiles
    constexpr int N = MI == 32 ? 8 : 32;
    using AccT = typename std::conditional<MI == 32, floatx16, floatx4>::type;
    AccT acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        acc[i] = AccT{0};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if constexpr (MI == 32)
                acc[i] = mfma32<IN>(a[i & 3], b[(i >> 2) & 3], acc[i]);
            else
                acc[i] = mfma16<IN>(a[i & 3], b[(i >> 2) & 3], acc[i]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int v = 0; v < (MI == 32 ? 16 : 4); ++v)
            s += acc[i][v];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// L2 fill probe.  Workgroup b runs on XCD b % 8 (round-robin dispatch).  The
// XCD's workgroups form `replicas` groups that each sweep the XCD's region
// once per pass; in a group, wave u (member m, wave w: u = 8m + w) takes the
// request-sized blocks u, u + 8*members, ...  Each wave keeps DEPTH requests
// in flight.  MODE 0: 16-byte loads straight into a 1 KiB LDS sink of the
// wave's own (the GEMM's copy form; nothing reads the sink); MODE 1: 16-byte
// loads into registers; MODE 2: 4-byte loads into registers.  The register
// forms XOR what they load into one value per thread and store it.
template <int MODE, int DEPTH>
__global__ void __launch_bounds__(512)
probe_fill(const uint8_t *buf, uint32_t footprint, int shared, int replicas, int64_t passes, float *sink,
           uint64_t *clocks)
{
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    __shared__ __attribute__((aligned(1024))) uint8_t lds_sink[8 * 1024];
    constexpr uint32_t REQ = MODE == 2 ? 4 : 16;     // bytes per lane
    constexpr uint32_t BLK = 64 * REQ;               // bytes per wave instruction
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int xcd = blockIdx.x % kNumXcd;
    const int j = blockIdx.x / kNumXcd;
    const int members = (int)(gridDim.x / kNumXcd) / replicas;
    const uint32_t u = (uint32_t)((j / replicas) * 8 + wave);
    const uint32_t stride = (uint32_t)members * 8u;
    const uint32_t nblk = footprint / BLK;
    const uint8_t *region = buf + (shared ? (size_t)0 : (size_t)xcd * footprint);
    const int64_t cnt = u < nblk ? (int64_t)((nblk - u + stride - 1) / stride) : 0;
    const int64_t total = cnt * passes;
    auto offset = [&](int64_t q) __attribute__((always_inline)) {
        return (u + (uint32_t)(q % cnt) * stride) * BLK + (uint32_t)lane * REQ;
    };
    uint32_t acc = 0;
    if constexpr (MODE == 0) {
        const i32x4 rs = make_rsrc4(region);
        const uint32_t lds_addr = (uint32_t)(uintptr_t)lds_sink + (uint32_t)wave * 1024u;
        // offsets are per lane here; dma16 adds 16*lane to the LDS address
        for (int64_t q = 0; q < total; ++q) {
            if (q >= DEPTH)
                wait_vmcnt<DEPTH - 1>();
            dma16(rs, lds_addr, offset(q), 0);
        }
        wait_vmcnt<0>();
    } else {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(region);
        using V = typename std::conditional<MODE == 1, u32x4, uint32_t>::type;
        V v[DEPTH];
        auto load = [&](int64_t q) __attribute__((always_inline)) {
            if constexpr (MODE == 1)
                return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, offset(q), 0, 0));
            else
                return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, offset(q), 0, 0);
        };
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if (d < total)
                v[d] = load(d);
        for (int64_t q = 0; q < total; q += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                if (q + d < total) {
                    if constexpr (MODE == 1)
                        acc ^= v[d][0] ^ v[d][1] ^ v[d][2] ^ v[d][3];
                    else
                        acc ^= v[d];
                    if (q + d + DEPTH < total)
                        v[d] = load(q + d + DEPTH);
                }
            }
        }
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = __builtin_bit_cast(float, acc);
    // the workgroup's shader-clock and 100 MHz-clock spans (thread 0's view)
    if (clocks != nullptr && threadIdx.x == 0) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        uint64_t *c = clocks + 4 * (int64_t)blockIdx.x;
        c[0] = t0;
        c[1] = t1;
        c[2] = r0;
        c[3] = r1;
    }
}

}  // namespace mpg

namespace {

template <int MODE>
hipError_t launch_fill(int depth, dim3 grid, hipStream_t s, const uint8_t *buf, uint32_t footprint,
                       int shared, int replicas, int64_t passes, float *sink, uint64_t *clocks)
{
    switch (depth) {
    case 1:
        hipLaunchKernelGGL((mpg::probe_fill<MODE, 1>), grid, dim3(512), 0, s, buf, footprint, shared, replicas,
                           passes, sink, clocks);
        break;
    case 2:
        hipLaunchKernelGGL((mpg::probe_fill<MODE, 2>), grid, dim3(512), 0, s, buf, footprint, shared, replicas,
                           passes, sink, clocks);
        break;
    case 4:
        hipLaunchKernelGGL((mpg::probe_fill<MODE, 4>), grid, dim3(512), 0, s, buf, footprint, shared, replicas,
                           passes, sink, clocks);
        break;
    case 8:
        hipLaunchKernelGGL((mpg::probe_fill<MODE, 8>), grid, dim3(512), 0, s, buf, footprint, shared, replicas,
                           passes, sink, clocks);
        break;
    default:
        hipLaunchKernelGGL((mpg::probe_fill<MODE, 16>), grid, dim3(512), 0, s, buf, footprint, shared, replicas,
                           passes, sink, clocks);
        break;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

int mpgemm_probe_mfma_layout(int shape, float *out, void *stream)
{
    if (shape != 32 && shape != 16)
        return MPGEMM_ECONFIG;
    if (out == nullptr)
        return MPGEMM_ENULL;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mpg::probe_mfma, dim3(1), dim3(64), 0,
                       reinterpret_cast<hipStream_t>(stream), out, shape);
    return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}

int mpgemm_probe_mfma_rate(int in_type, int shape, const uint16_t *ops, int64_t ops_len, int64_t iters,
                           int workgroups, float *out, int64_t out_len, void *stream)
{
    if ((in_type != MPGEMM_IN_F16 && in_type != MPGEMM_IN_BF16) || (shape != 32 && shape != 16))
        return MPGEMM_ECONFIG;
    if (ops == nullptr || out == nullptr)
        return MPGEMM_ENULL;
    if (ops_len < 4096 || iters < 0 || iters > (int64_t)1 << 24 || workgroups < 1 || workgroups > 65535 ||
        out_len < (int64_t)workgroups * 512)
        return MPGEMM_EDIM;
    (void)hipGetLastError();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)workgroups), block(512);
    if (in_type == MPGEMM_IN_F16) {
        if (shape == 32)
            hipLaunchKernelGGL((mpg::probe_mfma_rate<mpg::kInF16, 32>), grid, block, 0, s, ops, iters, out);
        else
            hipLaunchKernelGGL((mpg::probe_mfma_rate<mpg::kInF16, 16>), grid, block, 0, s, ops, iters, out);
    } else {
        if (shape == 32)
            hipLaunchKernelGGL((mpg::probe_mfma_rate<mpg::kInBF16, 32>), grid, block, 0, s, ops, iters, out);
        else
            hipLaunchKernelGGL((mpg::probe_mfma_rate<mpg::kInBF16, 16>), grid, block, 0, s, ops, iters, out);
    }
    return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}

int mpgemm_probe_fill(int mode, int depth, const void *buf, int64_t buf_bytes, int64_t footprint,
                      int shared, int replicas, int64_t passes, int workgroups, float *sink,
                      int64_t sink_len, uint64_t *clocks, int64_t clocks_len, void *stream)
{
    if (mode != MPGEMM_FILL_LDS16 && mode != MPGEMM_FILL_REG16 && mode != MPGEMM_FILL_REG4)
        return MPGEMM_ECONFIG;
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16)
        return MPGEMM_ECONFIG;
    if (buf == nullptr || sink == nullptr)
        return MPGEMM_ENULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return MPGEMM_EALIGN;
    if (workgroups < 8 || workgroups > 65535 || workgroups % 8 != 0 || replicas < 1 ||
        (workgroups / 8) % replicas != 0)
        return MPGEMM_EDIM;
    if (footprint <= 0 || footprint % 65536 != 0 || buf_bytes < 0 || buf_bytes >= ((int64_t)1 << 31) ||
        footprint > buf_bytes / (shared ? 1 : 8))
        return MPGEMM_EDIM;
    if (passes < 1 || passes > ((int64_t)1 << 20) || sink_len < (int64_t)workgroups * 512)
        return MPGEMM_EDIM;
    if (clocks != nullptr && clocks_len < (int64_t)workgroups * 4)
        return MPGEMM_EDIM;
    (void)hipGetLastError();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)workgroups);
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    const uint32_t fp = (uint32_t)footprint;
    hipError_t err;
    if (mode == MPGEMM_FILL_LDS16)
        err = launch_fill<0>(depth, grid, s, b, fp, shared, replicas, passes, sink, clocks);
    else if (mode == MPGEMM_FILL_REG16)
        err = launch_fill<1>(depth, grid, s, b, fp, shared, replicas, passes, sink, clocks);
    else
        err = launch_fill<2>(depth, grid, s, b, fp, shared, replicas, passes, sink, clocks);
    return err == hipSuccess ? MPGEMM_OK : MPGEMM_ELAUNCH;
}

}  // extern "C"
