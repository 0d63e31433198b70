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
// and the block scale is known to all 16 lanes without LDS.  The row's sum
// of squares is a per-thread fp32 sum, a 64-lane butterfly, and a fixed-order
// sum of the four wave totals through LDS, so every thread sees the same
// value and the result does not depend on scheduling.
//
// Bytes per row: 4H read (hidden + residual) + 4H read of the norm weight
// (cache-resident across rows) + 2H (bf16) + H (codes) + H/32 (scales)
// written: HBM-bound.

#include "device_common.h"
#include "kernels.h"

namespace mtpd {

template <int NSTEP>
__global__ __launch_bounds__(256) void norm_quant_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ residual,
    const float* __restrict__ gamma, float eps, int H,
    uint16_t* __restrict__ out_hidden, uint8_t* __restrict__ codes, float* __restrict__ scales)
{
    __shared__ float wave_sum[4];
    const int t = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * (size_t)H;
    const int KB = H >> 7;

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

    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(s[k][i], s[k][i], ss);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((t & 63) == 0) wave_sum[t >> 6] = ss;
    __syncthreads();
    const float total = (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
    const float rstd = (float)(1.0 / sqrt((double)total / (double)H + (double)eps));

#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 2048 + t * 8;
        if (c >= H) continue;   // uniform over each 16-thread scale block
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + c);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + c + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float y[8];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[i] = (s[k][i] * rstd) * g[i];
            amax = fmaxf(amax, fabsf(y[i]));
        }
        uint4 hb;
        hb.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
        hb.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
        hb.z = bf16_rne(y[4]) | (bf16_rne(y[5]) << 16);
        hb.w = bf16_rne(y[6]) | (bf16_rne(y[7]) << 16);
        *reinterpret_cast<uint4*>(out_hidden + base + c) = hb;

#pragma unroll
        for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        // RN_f32(amax / 448): the fp64 quotient rounds once more to fp32; a
        // quotient by 448 = 7 * 64 never lands on a false fp32 halfway point.
        const float scale = (float)((double)amax / 448.0);
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = scale > 0.f ? y[i] / scale : 0.f;   // correctly rounded fp32 quotient
            q[i] = fminf(fmaxf(v, -448.f), 448.f);
        }
        int lo = 0, hi = 0;
        lo = cvt_e4m3x2<false>(q[0], q[1], lo);
        lo = cvt_e4m3x2<true>(q[2], q[3], lo);
        hi = cvt_e4m3x2<false>(q[4], q[5], hi);
        hi = cvt_e4m3x2<true>(q[6], q[7], hi);
        *reinterpret_cast<uint2*>(codes + base + c) = make_uint2((uint32_t)lo, (uint32_t)hi);
        if ((t & 15) == 0) scales[(size_t)blockIdx.x * KB + (c >> 7)] = scale;
    }
}

hipError_t launch_norm_quant(const uint16_t* hidden, const uint16_t* residual, const float* gamma,
                             float eps, int64_t M, int64_t H, uint16_t* out_hidden, uint8_t* codes,
                             float* scales, hipStream_t stream)
{
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
