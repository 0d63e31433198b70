// Block-scaled FP8 LM head fused with a greedy argmax, for gfx950.
//
// The LM head consumes the packed activation as produced (E4M3 codes plus one
// fp32 scale per row per 128 columns) without unpacking it ("[Quant][MTP]
// Reuse packed FP8 logits inputs", Purpose and Dependencies), against an
// E4M3 weight with one fp32 scale per 128x128 block.  The greedy draft token
// is the local argmax over this weight's vocab rows, so logits never leave
// registers ("[Spec Decode][Perf] Fuse the MTP trailing all-reduce;
// local-argmax draft tokens", Summary).
//
// Mapping to CDNA4:
//  - One v_mfma_f32_16x16x128_f8f6f4 covers a 16x16 output tile over exactly
//    one 128-wide K scale block, so each MFMA result is an unscaled block
//    partial; the wave promotes it in fp32 as acc += p * (sa[row] * sw), the
//    same instruction sequence for every vocab row, so identical weight rows
//    give bit-identical logits wherever they sit.
//  - Operand fragments are loaded straight from global memory into VGPRs in
//    the MFMA layout: lane l holds row (l % 16) of the tile and the 32 K-bytes
//    {g*16 .. g*16+15} and {64+g*16 .. 64+g*16+15} of the block, g = l / 16.
//    A and B use the same K assignment, so the hardware's internal K order
//    does not matter.  Each weight row contributes one full 128-byte segment
//    per K block.  The next K block is loaded while the current one is in the
//    matrix core.
//  - A workgroup owns MT*16 activation rows x NT*16 vocab rows, all inside one
//    128-row weight-scale block.  Its S waves split K into S contiguous
//    ranges; partial accumulators meet in LDS and are summed in wave order,
//    so results do not depend on timing.  The activation scales of the row
//    tile are staged once in LDS, K-major, so each lane reads the 4 scales of
//    its 4 output rows with one 16-byte LDS load.
//  - Epilogue: the wave folds (logit, vocab index) into a u64 key whose
//    maximum is the largest logit and, on equal logits, the lowest index; a
//    16-lane shuffle reduction leaves one key per row, and one device-scope
//    atomicMax per (row, workgroup) merges workgroups.  The last workgroup
//    to finish (a device-scope completion counter) decodes the keys into
//    (max, index) and clears keys and counter for the next call.
//
// In the weight-streaming (decode) regime the cost is the weight read:
// V*H code bytes + V*H/16384*4 scale bytes per call.

#include <stdlib.h>

#include "device_common.h"
#include "kernels.h"

namespace mtpd {

__device__ __forceinline__ v8i load_frag(const uint8_t* p) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + 64);
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

__device__ __forceinline__ v4f mfma_e4m3(v8i a, v8i b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format selectors 0/0 = E4M3 for both operands; zero block scales select
    // the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <int MT, int NT, int S>
__global__ __launch_bounds__(64 * S) void lmhead_argmax_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int n_row_tiles, int total_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx,
    unsigned long long* __restrict__ keys, unsigned int* __restrict__ counter)
{
    constexpr int ROWS = MT * 16;
    constexpr int COLS = NT * 16;
    extern __shared__ float lds[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int KB = H >> 7;
    const int tile = xcd_contiguous((int)blockIdx.x, total_tiles);
    const int rt = tile % n_row_tiles;
    const int m0 = rt * ROWS;
    const int n0 = (tile / n_row_tiles) * COLS;
    const int vb = n0 >> 7;

    // activation scales of this row tile, K-major: sa_lds[kb * ROWS + r]
    float* sa_lds = lds;
    for (int e = threadIdx.x; e < KB * ROWS; e += 64 * S) {
        const int r = e / KB, kb = e - r * KB;
        const int m = min(m0 + r, n_rows - 1);
        const int a = row_index ? row_index[m] : m;
        sa_lds[kb * ROWS + r] = a_scales[(size_t)a * KB + kb];
    }

    const uint8_t* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = min(m0 + mt * 16 + (lane & 15), n_rows - 1);
        const int a = row_index ? row_index[m] : m;
        ap[mt] = a_codes + (size_t)a * H + (lane >> 4) * 16;
    }
    const uint8_t* wp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        wp[nt] = w_codes + (size_t)(n0 + nt * 16 + (lane & 15)) * H + (lane >> 4) * 16;
    const float* swp = w_scales + (size_t)vb * KB;

    __syncthreads();

    float acc[MT][NT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.f;

    const int kb0 = (wave * KB) / S;
    const int kb1 = ((wave + 1) * KB) / S;

    auto load = [&](v8i (&af)[MT], v8i (&wf)[NT], int kb) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wf[nt] = load_frag(wp[nt] + kb * kBlock);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[mt] = load_frag(ap[mt] + kb * kBlock);
    };
    auto compute = [&](const v8i (&af)[MT], const v8i (&wf)[NT], int kb) {
        const float sw = swp[kb];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float4 sa = *reinterpret_cast<const float4*>(&sa_lds[kb * ROWS + mt * 16 + 4 * (lane >> 4)]);
            const float f[4] = {sa.x * sw, sa.y * sw, sa.z * sw, sa.w * sw};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const v4f p = mfma_e4m3(af[mt], wf[nt]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(p[i], f[i], acc[mt][nt][i]);
            }
        }
    };

    v8i a0[MT], w0[NT], a1[MT], w1[NT];
    int kb = kb0;
    if (kb < kb1) load(a0, w0, kb);
    for (; kb + 1 < kb1; kb += 2) {
        load(a1, w1, kb + 1);
        compute(a0, w0, kb);
        if (kb + 2 < kb1) load(a0, w0, kb + 2);
        compute(a1, w1, kb + 1);
    }
    if (kb < kb1) compute(a0, w0, kb);

    if constexpr (S > 1) {
        float* part = lds + KB * ROWS;   // [(S-1)][MT*NT*4][64]
        constexpr int NE = MT * NT * 4;
        if (wave > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        part[((wave - 1) * NE + (mt * NT + nt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < S; ++w)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mt][nt][i] += part[((w - 1) * NE + (mt * NT + nt) * 4 + i) * 64 + lane];
    }

    // wave 0: per-row best key of this tile, merged across workgroups
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint64_t best = 0;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                best = u64_max(best, argmax_key(acc[mt][nt][i], (uint32_t)(n0 + nt * 16 + (lane & 15))));
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) best = u64_max(best, shfl_xor_u64(best, off));
            const int row = m0 + mt * 16 + 4 * (lane >> 4) + i;
            if ((lane & 15) == 0 && row < n_rows)
                atomicMax(&keys[row], (unsigned long long)best);
        }
    }

    __threadfence();
    unsigned int prev = 0;
    if (lane == 0) prev = atomicAdd(counter, 1u);
    prev = __shfl(prev, 0);
    if (prev != (unsigned int)(total_tiles - 1)) return;

    // last workgroup: every other workgroup's keys are visible
    __threadfence();
    for (int r = lane; r < n_rows; r += 64) {
        const uint64_t k = __hip_atomic_load(&keys[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        out_max[r] = key_value(k);
        out_idx[r] = key_index(k);
        __hip_atomic_store(&keys[r], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

namespace {

struct Tile {
    int mt, nt, s;
};

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

size_t lds_bytes(const Tile& t, int KB) {
    return (size_t)KB * t.mt * 16 * 4 + (size_t)(t.s - 1) * t.mt * t.nt * 4 * 64 * 4;
}

Tile choose_tile(int64_t n_rows, int64_t V, int64_t H) {
    Tile t;
    t.mt = n_rows <= 16 ? 1 : (n_rows <= 32 ? 2 : 4);
    t.nt = t.mt == 1 ? 2 : 4;
    const int KB = (int)(H / kBlock);
    // optional launch-shape override for tuning sweeps: MTPD_LMHEAD_TILE="nt,s"
    int env_nt = 0, env_s = 0;
    if (const char* e = getenv("MTPD_LMHEAD_TILE")) {
        if (sscanf(e, "%d,%d", &env_nt, &env_s) != 2) env_nt = env_s = 0;
    }
    if (env_nt == 1 || env_nt == 2 || env_nt == 4) t.nt = env_nt;
    const int64_t row_tiles = (n_rows + t.mt * 16 - 1) / (t.mt * 16);
    const int64_t tiles = row_tiles * (V / (t.nt * 16));
    const int64_t want_waves = 8LL * device_cus();
    t.s = 1;
    while (t.s < 8 && tiles * t.s < want_waves && 2 * t.s <= KB) t.s *= 2;
    if (env_s == 1 || env_s == 2 || env_s == 4 || env_s == 8) t.s = env_s;
    // 512-thread workgroups cap a thread at 256 registers: only small tiles fit
    if (t.s == 8 && t.mt * t.nt > 4) t.s = 4;
    while (t.s > 1 && lds_bytes(t, KB) > 64 * 1024) t.s /= 2;
    return t;
}

template <int MT, int NT, int S>
hipError_t launch_t(const LmheadArgs& a, hipStream_t stream) {
    const int KB = (int)(a.H / kBlock);
    const int64_t row_tiles = (a.n_rows + MT * 16 - 1) / (MT * 16);
    const int64_t tiles = row_tiles * (a.V / (NT * 16));
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = lds_bytes(Tile{MT, NT, S}, KB);
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(a.workspace);
    unsigned int* counter = reinterpret_cast<unsigned int*>(keys + a.n_rows);
    hipLaunchKernelGGL((lmhead_argmax_kernel<MT, NT, S>), dim3((unsigned)tiles), dim3(64 * S), lds, stream,
                       a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales, (int)a.H,
                       (int)row_tiles, (int)tiles, a.out_max, a.out_idx, keys, counter);
    return hipGetLastError();
}

template <int MT, int NT>
hipError_t launch_s(const LmheadArgs& a, int s, hipStream_t stream) {
    switch (s) {
        case 1: return launch_t<MT, NT, 1>(a, stream);
        case 2: return launch_t<MT, NT, 2>(a, stream);
        case 4: return launch_t<MT, NT, 4>(a, stream);
        case 8:
            if constexpr (MT * NT <= 4) return launch_t<MT, NT, 8>(a, stream);
            break;
    }
    return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_n(const LmheadArgs& a, int nt, int s, hipStream_t stream) {
    switch (nt) {
        case 1: return launch_s<MT, 1>(a, s, stream);
        case 2: return launch_s<MT, 2>(a, s, stream);
        case 4: return launch_s<MT, 4>(a, s, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_lmhead_argmax(const LmheadArgs& a, hipStream_t stream) {
    const Tile t = choose_tile(a.n_rows, a.V, a.H);
    switch (t.mt) {
        case 1: return launch_n<1>(a, t.nt, t.s, stream);
        case 2: return launch_n<2>(a, t.nt, t.s, stream);
        case 4: return launch_n<4>(a, t.nt, t.s, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mtpd
