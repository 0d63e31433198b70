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

// The dispatcher places workgroup b on XCD (b mod 8).  Give each XCD a
// contiguous range of logical tile ids so tiles that share operands land on
// the same XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int b, int total) {
    const int per = total >> 3, rem = total & 7;
    const int xcd = b & 7, k = b >> 3;
    return xcd * per + (xcd < rem ? xcd : rem) + k;
}

}  // namespace mtpd
