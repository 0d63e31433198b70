// Residual add + RMSNorm + dual output (bf16 recycled hidden, packed FP8
// activation) for gfx950.
//
// The step is the MTP layer's final norm fused with packed FP8 quantization
// for the shared LM head ("[Quant][MTP] Reuse packed FP8 logits inputs",
// Purpose); the norm statistic accumulates in fp32 ("[Spec Decode][Perf]
// Fuse the MTP trailing all-reduce; local-argmax draft tokens", Accuracy).
//
// Layout: one 256-thread workgroup per row.  Thread t owns the 8 contiguous
// columns step*2048 + 8t of each 2048-column step, loaded as one 16-byte
// bf16 vector from hidden and one from residual, and kept in registers (at
// most 8 steps, H <= 16384).  Sixteen consecutive threads cover exactly one
// 128-column scale block, so the block amax is a 16-lane shuffle reduction
// and the block scale is known to all 16 lanes without LDS (DPP moves inside
// the lane row).  The row's sum of squares is a per-thread fp32 sum, a wave
// sum with one fixed association (DPP inside each 16-lane row, then the four
// row sums), and a fixed-order sum of the four wave totals through LDS, so
// every thread sees the same value and the result does not depend on
// scheduling.
//
// Bytes per row: 4H read (hidden + residual) + 4H read of the norm weight
// (cache-resident across rows) + 2H (bf16) + H (codes) + H/32 (scales)
// written: HBM-bound.

#include "device_common.h"
#include "kernels.h"

namespace mtpd {

// The norm and the two outputs for one row, from the fp32 norm input s held
// in registers (thread t owns columns step*2048 + 8t .. +7; zero past H).
template <int NSTEP>
__device__ __forceinline__ void norm_quant_finish(const float (&s)[NSTEP][8], const float* __restrict__ gamma,
                                                  float eps, int H, size_t row, float* wave_sum,
                                                  uint16_t* __restrict__ out_hidden, uint8_t* __restrict__ codes,
                                                  float* __restrict__ scales)
{
    const int t = threadIdx.x;
    const size_t base = row * (size_t)H;
    const int KB = H >> 7;

    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(s[k][i], s[k][i], ss);
    ss = wave_sum_f32(ss);
    if ((t & 63) == 0) wave_sum[t >> 6] = ss;
    __syncthreads();
    const float total = (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
    const float rstd = (float)(1.0 / sqrt((double)total / (double)H + (double)eps));

    // every group computed (columns past H hold s = 0 and read a clamped
    // norm weight; they fill whole 128-column blocks, which are not stored)
    float y[NSTEP][8];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = min(k * 2048 + t * 8, H - 8);
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + c);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + c + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[k][i] = (s[k][i] * rstd) * g[i];
    }
    float scale[NSTEP];
    uint2 code[NSTEP];
    quant_groups<NSTEP>(y, scale, code);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 2048 + t * 8;
        if (c >= H) continue;   // uniform over each 16-thread scale block
        *reinterpret_cast<uint4*>(out_hidden + base + c) = pack_bf16x8(y[k]);
        *reinterpret_cast<uint2*>(codes + base + c) = code[k];
        if ((t & 15) == 0) scales[row * KB + (c >> 7)] = scale[k];
    }
}

// Adds the 8 bf16 values of v to s (fp32, one rounding per element).
__device__ __forceinline__ void add_bf16x8(float (&s)[8], const uint4 v) {
    s[0] += bf16_lo(v.x);
    s[1] += bf16_hi(v.x);
    s[2] += bf16_lo(v.y);
    s[3] += bf16_hi(v.y);
    s[4] += bf16_lo(v.z);
    s[5] += bf16_hi(v.z);
    s[6] += bf16_lo(v.w);
    s[7] += bf16_hi(v.w);
}

template <int NSTEP>
__global__ __launch_bounds__(256) void norm_quant_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ residual,
    const float* __restrict__ gamma, float eps, int H,
    uint16_t* __restrict__ out_hidden, uint8_t* __restrict__ codes, float* __restrict__ scales)
{
    __shared__ float wave_sum[4];
    const int t = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * (size_t)H;

    float s[NSTEP][8];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 2048 + t * 8;
        if (c < H) {
            const uint4 hv = *reinterpret_cast<const uint4*>(hidden + base + c);
            const uint4 rv = *reinterpret_cast<const uint4*>(residual + base + c);
            s[k][0] = bf16_lo(hv.x) + bf16_lo(rv.x);
            s[k][1] = bf16_hi(hv.x) + bf16_hi(rv.x);
            s[k][2] = bf16_lo(hv.y) + bf16_lo(rv.y);
            s[k][3] = bf16_hi(hv.y) + bf16_hi(rv.y);
            s[k][4] = bf16_lo(hv.z) + bf16_lo(rv.z);
            s[k][5] = bf16_hi(hv.z) + bf16_hi(rv.z);
            s[k][6] = bf16_lo(hv.w) + bf16_lo(rv.w);
            s[k][7] = bf16_hi(hv.w) + bf16_hi(rv.w);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s[k][i] = 0.f;
        }
    }
    norm_quant_finish<NSTEP>(s, gamma, eps, H, blockIdx.x, wave_sum, out_hidden, codes, scales);
}

// ---------------------------------------------------------------------------
// The same step with one wavefront per row (four rows per 256-thread
// workgroup), for measurement against the workgroup per row above (plan
// override "norm_quant" = "wave").  Lane l owns columns k * 512 + 8l .. + 7
// of each 512-column step (H <= 8192: at most 16 steps in registers);
// sixteen lanes still cover one 128-column scale block.  The row's sum of
// squares is the per-lane fp32 sum and one wave sum, with no exchange
// between waves, so its association differs from the kernel above: results
// agree with it to rounding, not bit for bit.
// ---------------------------------------------------------------------------

template <int NSTEP>
__global__ __launch_bounds__(256) void norm_quant_wave_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ residual,
    const float* __restrict__ gamma, float eps, int H, int M,
    uint16_t* __restrict__ out_hidden, uint8_t* __restrict__ codes, float* __restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int row = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (row >= M) return;   // the whole wave: nothing below synchronizes across waves
    const size_t base = (size_t)row * (size_t)H;
    const int KB = H >> 7;

    float s[NSTEP][8];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 512 + lane * 8;
        if (c < H) {
            const uint4 hv = *reinterpret_cast<const uint4*>(hidden + base + c);
            const uint4 rv = *reinterpret_cast<const uint4*>(residual + base + c);
            s[k][0] = bf16_lo(hv.x) + bf16_lo(rv.x);
            s[k][1] = bf16_hi(hv.x) + bf16_hi(rv.x);
            s[k][2] = bf16_lo(hv.y) + bf16_lo(rv.y);
            s[k][3] = bf16_hi(hv.y) + bf16_hi(rv.y);
            s[k][4] = bf16_lo(hv.z) + bf16_lo(rv.z);
            s[k][5] = bf16_hi(hv.z) + bf16_hi(rv.z);
            s[k][6] = bf16_lo(hv.w) + bf16_lo(rv.w);
            s[k][7] = bf16_hi(hv.w) + bf16_hi(rv.w);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s[k][i] = 0.f;
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(s[k][i], s[k][i], ss);
    ss = wave_sum_f32(ss);
    const float rstd = (float)(1.0 / sqrt((double)ss / (double)H + (double)eps));
    // y over s in place (columns past H hold s = 0 and read a clamped norm
    // weight; they fill whole 128-column blocks, which are not stored)
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = min(k * 512 + lane * 8, H - 8);
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + c);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + c + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) s[k][i] = (s[k][i] * rstd) * g[i];
    }
    float scale[NSTEP];
    uint2 code[NSTEP];
    quant_groups<NSTEP>(s, scale, code);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 512 + lane * 8;
        if (c >= H) continue;   // uniform over each 16-lane scale block
        *reinterpret_cast<uint4*>(out_hidden + base + c) = pack_bf16x8(s[k]);
        *reinterpret_cast<uint2*>(codes + base + c) = code[k];
        if ((lane & 15) == 0) scales[(size_t)row * KB + (c >> 7)] = scale[k];
    }
}

// ---------------------------------------------------------------------------
// The same step with the MTP layer's trailing all-reduce folded in: the norm
// input is the sum of P row-parallel partial outputs plus the residual
// ("[Spec Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax draft
// tokens", Summary: the all-reduce and the RMSNorm run as one fused step;
// Accuracy: fp32 accumulation).  Here the P partials are device buffers on
// this GPU standing in for the peers' outputs (a one-shot all-reduce reads
// each peer's buffer once); the transport between GPUs is not part of it.
//
//   s = ((p_0 + p_1) + ... + p_{P-1}) + residual      fp32, in partial order
//
// PMAX >= P loads are issued per 2048-column step before any add (addresses
// of partials past P repeat partial 0 and their values are not added), so a
// row's whole input is in flight at once.  With P == 1 the result is
// bit-identical to norm_quant_kernel on (p_0, residual).
//
// Bytes per row: 2H (P + 1) read + 4H of norm weight (cache-resident) +
// 3H + H/32 written.
// ---------------------------------------------------------------------------

template <int NSTEP, int PMAX>
__global__ __launch_bounds__(256) void allreduce_norm_quant_kernel(
    PartialPtrs parts, const uint16_t* __restrict__ residual,
    const float* __restrict__ gamma, float eps, int H,
    uint16_t* __restrict__ out_hidden, uint8_t* __restrict__ codes, float* __restrict__ scales)
{
    __shared__ float wave_sum[4];
    const int t = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * (size_t)H;
    const int P = parts.n;

    float s[NSTEP][8];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 2048 + t * 8;
        if (c < H) {
            uint4 pv[PMAX];
#pragma unroll
            for (int q = 0; q < PMAX; ++q)
                pv[q] = *reinterpret_cast<const uint4*>(parts.p[q < P ? q : 0] + base + c);
            const uint4 rv = *reinterpret_cast<const uint4*>(residual + base + c);
            s[k][0] = bf16_lo(pv[0].x);
            s[k][1] = bf16_hi(pv[0].x);
            s[k][2] = bf16_lo(pv[0].y);
            s[k][3] = bf16_hi(pv[0].y);
            s[k][4] = bf16_lo(pv[0].z);
            s[k][5] = bf16_hi(pv[0].z);
            s[k][6] = bf16_lo(pv[0].w);
            s[k][7] = bf16_hi(pv[0].w);
#pragma unroll
            for (int q = 1; q < PMAX; ++q)
                if (q < P) add_bf16x8(s[k], pv[q]);
            add_bf16x8(s[k], rv);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s[k][i] = 0.f;
        }
    }
    norm_quant_finish<NSTEP>(s, gamma, eps, H, blockIdx.x, wave_sum, out_hidden, codes, scales);
}

hipError_t launch_norm_quant(const uint16_t* hidden, const uint16_t* residual, const float* gamma,
                             float eps, int64_t M, int64_t H, uint16_t* out_hidden, uint8_t* codes,
                             float* scales, hipStream_t stream)
{
    if (plan_override().norm_quant == 1 && H <= 8192) {
        const int nw = (int)((H + 511) / 512);
        const dim3 grid((unsigned)((M + 3) / 4)), block(256);
#define MTPD_NQW_CASE(N)                                                                                   \
    case N:                                                                                                \
        hipLaunchKernelGGL(norm_quant_wave_kernel<N>, grid, block, 0, stream, hidden, residual, gamma, eps, \
                           (int)H, (int)M, out_hidden, codes, scales);                                     \
        break;
        switch (nw) {
            MTPD_NQW_CASE(1) MTPD_NQW_CASE(2) MTPD_NQW_CASE(3) MTPD_NQW_CASE(4)
            MTPD_NQW_CASE(5) MTPD_NQW_CASE(6) MTPD_NQW_CASE(7) MTPD_NQW_CASE(8)
            MTPD_NQW_CASE(9) MTPD_NQW_CASE(10) MTPD_NQW_CASE(11) MTPD_NQW_CASE(12)
            MTPD_NQW_CASE(13) MTPD_NQW_CASE(14) MTPD_NQW_CASE(15) MTPD_NQW_CASE(16)
            default:
                return hipErrorInvalidValue;
        }
#undef MTPD_NQW_CASE
        return hipGetLastError();
    }
    const int nstep = (int)((H + 2047) / 2048);
    const dim3 grid((unsigned)M), block(256);
#define MTPD_NQ_CASE(N)                                                                              \
    case N:                                                                                          \
        hipLaunchKernelGGL(norm_quant_kernel<N>, grid, block, 0, stream, hidden, residual, gamma,   \
                           eps, (int)H, out_hidden, codes, scales);                                 \
        break;
    switch (nstep) {
        MTPD_NQ_CASE(1)
        MTPD_NQ_CASE(2)
        MTPD_NQ_CASE(3)
        MTPD_NQ_CASE(4)
        MTPD_NQ_CASE(5)
        MTPD_NQ_CASE(6)
        MTPD_NQ_CASE(7)
        MTPD_NQ_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef MTPD_NQ_CASE
    return hipGetLastError();
}

}  // namespace mtpd

namespace mtpd {

hipError_t launch_allreduce_norm_quant(const PartialPtrs& parts, const uint16_t* residual, const float* gamma,
                                       float eps, int64_t M, int64_t H, uint16_t* out_hidden, uint8_t* codes,
                                       float* scales, hipStream_t stream)
{
    if (parts.n < 1 || parts.n > kMaxPartials) return hipErrorInvalidValue;
    const int nstep = (int)((H + 2047) / 2048);
    const int pmax = parts.n <= 2 ? 2 : parts.n <= 4 ? 4 : parts.n <= 8 ? 8 : 16;
    const dim3 grid((unsigned)M), block(256);
#define MTPD_AR_CASE(N, Q)                                                                                \
    if (nstep == N && pmax == Q) {                                                                        \
        hipLaunchKernelGGL((allreduce_norm_quant_kernel<N, Q>), grid, block, 0, stream, parts, residual,   \
                           gamma, eps, (int)H, out_hidden, codes, scales);                                \
        return hipGetLastError();                                                                         \
    }
#define MTPD_AR_STEPS(Q) \
    MTPD_AR_CASE(1, Q) MTPD_AR_CASE(2, Q) MTPD_AR_CASE(3, Q) MTPD_AR_CASE(4, Q) \
    MTPD_AR_CASE(5, Q) MTPD_AR_CASE(6, Q) MTPD_AR_CASE(7, Q) MTPD_AR_CASE(8, Q)
    MTPD_AR_STEPS(2)
    MTPD_AR_STEPS(4)
    MTPD_AR_STEPS(8)
    MTPD_AR_STEPS(16)
#undef MTPD_AR_STEPS
#undef MTPD_AR_CASE
    return hipErrorInvalidValue;
}

}  // namespace mtpd
