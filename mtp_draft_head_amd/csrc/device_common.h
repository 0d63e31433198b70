// Device helpers shared by the gfx950 kernels of libmtpd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mtpd {

constexpr int kWave = 64;     // CDNA wavefront

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> two OCP E4M3FN codes in one 16-bit half of `old` (x in the
// lower byte, y in the upper), via the gfx950 hardware conversion (round to
// nearest even).  HIGH selects the upper 16 bits.  Inputs must already be
// clamped to +-448.
template <bool HIGH>
__device__ __forceinline__ int cvt_e4m3x2(float x, float y, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(x, y, old, HIGH);
}

// Eight fp32 values -> eight bf16 (round to nearest even), in column order.
__device__ __forceinline__ uint4 pack_bf16x8(const float (&y)[8]) {
    uint4 hb;
    hb.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
    hb.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
    hb.z = bf16_rne(y[4]) | (bf16_rne(y[5]) << 16);
    hb.w = bf16_rne(y[6]) | (bf16_rne(y[7]) << 16);
    return hb;
}

// Order-preserving map of an fp32 logit to u32 (-0 folded onto +0), packed
// with the vocab index so that the u64 maximum is the largest logit and,
// among equal logits, the lowest index.
__device__ __forceinline__ uint64_t argmax_key(float z, uint32_t idx) {
    uint32_t u = __float_as_uint(z);
    if (u == 0x80000000u) u = 0u;
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ float key_value(uint64_t k) {
    uint32_t ord = (uint32_t)(k >> 32);
    uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
}

__device__ __forceinline__ int32_t key_index(uint64_t k) {
    return (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t u64_min(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, mask);
    hi = __shfl_xor(hi, mask);
    return ((uint64_t)hi << 32) | lo;
}

// DPP moves inside each 16-lane row (gfx9 dpp_ctrl encodings): 0xB1 quad_perm
// [1,0,3,2] (lane ^ 1), 0x4E quad_perm [2,3,0,1] (lane ^ 2), 0x141
// row_half_mirror (lane i of each 8-lane half takes lane 7 - i), 0x140
// row_mirror (lane i takes lane 15 - i).  Each is one VALU operand modifier
// instead of an LDS round trip, and never reads outside the row, so a row
// that is entirely active gives the same result whatever the other rows do.
//
// The empty asm after each move pins it where every lane runs it: the
// compiler otherwise may recompute a move inside a branch it makes for a
// select, where lanes outside the branch are off and read as zero.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    int r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
    asm volatile("" : "+v"(r));
    return __int_as_float(r);
}

// Maximum over each 16-lane row, in every lane of the row (exact in any
// order).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    return fmaxf(v, dpp_f32<0x140>(v));
}

// Unsigned minimum over each 16-lane row, in every lane of the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    int r = __builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    asm volatile("" : "+v"(r));
    return (uint32_t)r;
}
__device__ __forceinline__ uint32_t row16_min_u32(uint32_t v) {
    v = min(v, dpp_u32<0xB1>(v));
    v = min(v, dpp_u32<0x4E>(v));
    v = min(v, dpp_u32<0x141>(v));
    return min(v, dpp_u32<0x140>(v));
}

// u64 maximum over each 16-lane row, in every lane of the row.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    asm volatile("" : "+v"(lo), "+v"(hi));
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
    v = u64_max(v, dpp_u64<0xB1>(v));
    v = u64_max(v, dpp_u64<0x4E>(v));
    v = u64_max(v, dpp_u64<0x141>(v));
    return u64_max(v, dpp_u64<0x140>(v));
}

// Sum over the 64 lanes of a fully active wave with one fixed association:
// lane pairs, then quads, then the two quads of each half-row, the two halves
// of each row (each step adds two partial sums of the same lanes, so the
// lanes of a group agree: fp addition commutes), and the four row sums as
// (r0 + r1) + (r2 + r3).  Wave-uniform result.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// E4M3 codes of eight values of one 128-column block whose scale is
// scale = RN_f32(amax / 448): code = E4M3(RN_f32(y / scale)) saturated to
// +-448, ties to even, a zero quotient keeping the sign of y; a zero scale
// gives +0 codes.
//
// For scale in [2^-60, 2^60] the quotient comes from one correctly rounded
// reciprocal r = RN(1/scale) per block: q0 = RN(y r), the exact remainder
// e = y - scale q0 (one fma), and RN(q0 + e r), which is the correctly
// rounded quotient by Markstein's theorem (r within half an ulp of 1/scale,
// q0 within one ulp of the quotient; the range keeps r, q0 and e clear of
// overflow and underflow wherever the quotient reaches the E4M3 range).
// Three operations per value instead of a full division; other scales take
// the full division.
__device__ __forceinline__ bool quant_fast_range(float scale) { return scale >= 0x1p-60f && scale <= 0x1p60f; }

__device__ __forceinline__ uint2 pack_e4m3x8(float (&q)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(q[i], -448.f, 448.f);
    int lo = 0, hi = 0;
    lo = cvt_e4m3x2<false>(q[0], q[1], lo);
    lo = cvt_e4m3x2<true>(q[2], q[3], lo);
    hi = cvt_e4m3x2<false>(q[4], q[5], hi);
    hi = cvt_e4m3x2<true>(q[6], q[7], hi);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// quant_fast_range(scale) must hold
__device__ __forceinline__ uint2 quant_e4m3x8_fast(const float (&y)[8], float scale) {
    const float r = 1.0f / scale;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q0 = y[i] * r;
        const float e = fmaf(-scale, q0, y[i]);
        q[i] = copysignf(fmaf(e, r, q0), y[i]);
    }
    return pack_e4m3x8(q);
}

__device__ __forceinline__ uint2 quant_e4m3x8_div(const float (&y)[8], float scale) {
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = scale > 0.f ? y[i] / scale : 0.f;
    return pack_e4m3x8(q);
}

// One thread's share of a row's packing: NSTEP groups of 8 columns, each
// inside one 128-column block whose 16 lanes form a DPP row.  Per group: the
// block amax (row16_max), scale = RN_f32(amax / 448) (the fp64 quotient
// rounds once more to fp32; a quotient by 448 = 7 * 64 never lands on a false
// fp32 halfway point), and the codes.  Straight-line over the groups (the
// rare full divisions come after), so their latency chains interleave.
template <int NSTEP>
__device__ __forceinline__ void quant_groups(const float (&y)[NSTEP][8], float (&scale)[NSTEP],
                                             uint2 (&code)[NSTEP]) {
    bool slow = false;
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[k][i]));
        amax = row16_max(amax);
        scale[k] = (float)((double)amax / 448.0);
        code[k] = quant_e4m3x8_fast(y[k], scale[k]);
        slow |= !quant_fast_range(scale[k]);
    }
    if (slow) {
#pragma unroll
        for (int k = 0; k < NSTEP; ++k)
            if (!quant_fast_range(scale[k])) code[k] = quant_e4m3x8_div(y[k], scale[k]);
    }
}

// The dispatcher places workgroup b on XCD (b mod 8).  Give each XCD a
// contiguous range of logical tile ids so tiles that share operands land on
// the same XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int b, int total) {
    const int per = total >> 3, rem = total & 7;
    const int xcd = b & 7, k = b >> 3;
    return xcd * per + (xcd < rem ? xcd : rem) + k;
}

}  // namespace mtpd
