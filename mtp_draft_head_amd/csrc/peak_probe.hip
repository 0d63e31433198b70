// Measured achievable peaks of the two units the LM head is bound by, for
// the benchmark's roofline beside the published ones: a streaming read of a
// device buffer (HBM, the decode regime) and a register-only loop of the FP8
// MFMA the LM-head kernels issue (the matrix cores, the compute regime).
// Built as its own library (libmtpd_peaks.so); the tail's path never calls it.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// Workgroup b reads 16-byte vectors [b * per_wg, (b + 1) * per_wg) of src,
// kReadUnroll loads in flight per lane, with the non-temporal policy of the
// LM head's weight copies; every lane folds what it read into one word and
// stores it, so no load is dead.
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const u32x4* __restrict__ src, uint64_t n_vec,
                                                                   uint64_t per_wg, unsigned* __restrict__ sink) {
    const uint64_t b0 = (uint64_t)blockIdx.x * per_wg;
    const uint64_t e = b0 + per_wg < n_vec ? b0 + per_wg : n_vec;
    unsigned acc = 0;
    for (uint64_t i = b0 + threadIdx.x; i < e; i += (uint64_t)kReadThreads * kReadUnroll) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) {
            const uint64_t k = i + (uint64_t)j * kReadThreads;
            v[j] = k < e ? __builtin_nontemporal_load(&src[k]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    sink[(uint64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

constexpr int kChains = 8;   // independent accumulators per wave (covers the MFMA latency)

// Each wave issues iters * kChains 16x16x128 E4M3 MFMAs on register
// operands (unscaled form, as in the LM-head kernels), kChains independent
// accumulations deep, and stores the sums so nothing is dead.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 ^ (lane << (i & 3));   // codes near 1.0
        b[i] = 0x30303030 ^ (i << 8);
    }
    v4f c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j)
            c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same loop on operands that look like real data: each lane loads two
// random operand pairs (words: grid * 256 * 32 u32) and the MFMAs alternate
// between them, so the multiplier inputs change from one instruction to the
// next as they do in the LM-head kernels (the matrix cores draw more power on
// such operands than on the near-constant ones above, and the clock follows).
__global__ __launch_bounds__(256) void mfma_loop_random_kernel(int iters, const uint32_t* __restrict__ words,
                                                               float* __restrict__ out) {
    const uint32_t* w = words + ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 32;
    v8i a0, b0, a1, b1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0[i] = (int)w[i];
        b0[i] = (int)w[8 + i];
        a1[i] = (int)w[16 + i];
        b1[i] = (int)w[24 + i];
    }
    v4f c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j)
            c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(j & 1 ? a1 : a0, j & 1 ? b1 : b0, c[j], 0, 0, 0, 0,
                                                                    0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16, src 16-byte aligned) by `grid`
// workgroups of 256 threads; sink: grid * 256 u32 of device memory.
int mtpd_peak_read(const void* src, uint64_t bytes, int grid, unsigned* sink, void* stream) {
    if (!src || !sink || grid < 1 || bytes % 16 || (uintptr_t)src % 16) return 1;
    const uint64_t n_vec = bytes / 16;
    const uint64_t per_wg = (n_vec + grid - 1) / grid;
    hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(kReadThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, n_vec, per_wg, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// FP8 MFMA loop: grid workgroups of 256 threads, iters iterations of 8 MFMAs
// per wave; out: grid * 256 floats.  Flops = grid * 4 * iters * 8 * 65536.
int mtpd_peak_mfma(int iters, int grid, float* out, void* stream) {
    if (!out || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The loop on random operands: words holds grid * 256 * 32 u32 of device
// memory (random E4M3 codes; the caller keeps NaN codes out, as the packing
// never produces them).
int mtpd_peak_mfma_random(int iters, int grid, const uint32_t* words, float* out, void* stream) {
    if (!out || !words || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_loop_random_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, words, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
