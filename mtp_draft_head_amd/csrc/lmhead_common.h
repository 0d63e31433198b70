// Pieces shared by the LM-head kernels: MFMA fragment helpers and the
// cross-workgroup argmax protocol.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace mtpd {

// 32 K-bytes of one 128-wide K block for an MFMA operand: lane l takes row
// (l % 16) of the 16-row tile (p already points at that row, at K-byte
// (l / 16) * 16 of the block) and the bytes at +0 and +64.
__device__ __forceinline__ v8i load_frag(const uint8_t* p) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + 64);
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

__device__ __forceinline__ v8i make_frag(uint4 lo, uint4 hi) {
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

// 16x16 tile over one 128-wide K block, E4M3 x E4M3 -> fp32, unscaled.
__device__ __forceinline__ v4f mfma_e4m3(v8i a, v8i b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format selectors 0/0 = E4M3 for both operands; zero block scales select
    // the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

typedef const float __attribute__((address_space(4)))* const_f32_ptr;

// Wave-uniform load through the scalar cache (the table is read-only for the
// whole kernel), so it never waits behind the vector-memory queue.
__device__ __forceinline__ float scalar_load(const float* p, int i) {
    return ((const_f32_ptr)p)[i];
}

// ---------------------------------------------------------------------------
// Cross-workgroup argmax.
//
// Workspace (zero between calls; layout in kernels.h):
//   keys      P partitions of n_rows u64 keys, slot (p, r) at
//             (p * n_rows + r) * stride: tile t merges its per-row best key
//             into partition t % P, and with stride 16 every slot is its own
//             128-byte line.  Atomics on one line serialize at the memory side
//             (about 12 ns each), so this keeps every line's queue short.
//   counters  kArriveGroups group counters (tile t arrives at t % groups) and
//             one top counter, each on its own 128-byte line
// Every cross-workgroup access is an atomic performed at the device's
// coherence point; ordering comes from data dependencies on returned values,
// not from cache-flushing fences.
// ---------------------------------------------------------------------------

constexpr int kCounterStride = 32;   // u32s per 128-byte line

struct ArgmaxWs {
    unsigned long long* keys;
    unsigned int* counters;
    int P;        // partitions, a power of two
    int stride;   // u64s between consecutive slots
};

__device__ __forceinline__ uint64_t merge_key(const ArgmaxWs& ws, int n_rows, int tile, int row, uint64_t key) {
    const size_t slot = ((size_t)(tile & (ws.P - 1)) * (size_t)n_rows + (size_t)row) * (size_t)ws.stride;
    return __hip_atomic_fetch_max(&ws.keys[slot], (unsigned long long)key, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// A value that is never nonzero for a returned key (a key naming a vocab
// index above 2^32 - 2^17, while V < 2^31) but that the compiler cannot
// prove zero: adding it to a counter increment makes the increment wait for
// the key update's return.
__device__ __forceinline__ unsigned int never_nonzero(uint64_t returned) {
    return ((uint32_t)(returned >> 32) == 0xFFFFFFFFu && (uint32_t)returned == 0x0001E240u) ? 1u : 0u;
}

// One lane per workgroup, after its key merges have returned (dep carries
// that dependency).  True for exactly one workgroup: the last to arrive.
__device__ __forceinline__ bool arrive(const ArgmaxWs& ws, int tile, int total_tiles, unsigned int dep) {
    constexpr int G = kArriveGroups;
    const int g = tile % G;
    const unsigned int group_size = (unsigned int)(total_tiles / G + (g < total_tiles % G ? 1 : 0));
    const unsigned int prev = __hip_atomic_fetch_add(&ws.counters[g * kCounterStride], 1u + dep, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
    if (prev != group_size - 1) return false;
    const unsigned int groups = total_tiles < G ? (unsigned int)total_tiles : (unsigned int)G;
    const unsigned int prev2 = __hip_atomic_fetch_add(&ws.counters[G * kCounterStride], 1u + never_nonzero(prev),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return prev2 == groups - 1;
}

// The same with one counter for the whole launch: one round trip fewer, but
// every arrival queues on one line, so for grids of a few hundred
// workgroups whose arrivals spread out in time.
__device__ __forceinline__ bool arrive_flat(const ArgmaxWs& ws, int total, unsigned int dep) {
    const unsigned int prev = __hip_atomic_fetch_add(&ws.counters[kArriveGroups * kCounterStride], 1u + dep,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return prev == (unsigned int)total - 1;
}

// The last workgroup (all NTHREADS threads): reduce the P partitions of every
// row, decode (max, index), and leave keys and counters zero.  red: LDS
// scratch of NTHREADS u64.
template <int NTHREADS>
__device__ void finalize_argmax(const ArgmaxWs& ws, int n_rows, float* __restrict__ out_max,
                                int32_t* __restrict__ out_idx, unsigned long long* red) {
    const int t = threadIdx.x;
    // every arrival of this launch has been counted: the counters can be
    // cleared now, their stores in flight beside the key exchanges below
    if (t <= kArriveGroups)
        __hip_atomic_store(&ws.counters[t * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int r0 = 0; r0 < n_rows; r0 += NTHREADS) {
        const int nr = min(NTHREADS, n_rows - r0);
        red[t] = 0;
        __syncthreads();
        const int npairs = ws.P * nr;
        for (int base = 0; base < npairs; base += NTHREADS * 16) {
            uint64_t k[16];
            int rr[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int e = base + u * NTHREADS + t;
                rr[u] = -1;
                k[u] = 0;
                if (e < npairs) {
                    const int p = e / nr, r = e - p * nr;
                    rr[u] = r;
                    k[u] = __hip_atomic_exchange(&ws.keys[((size_t)p * n_rows + r0 + r) * (size_t)ws.stride], 0ull,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (rr[u] >= 0) atomicMax(&red[rr[u]], (unsigned long long)k[u]);
        }
        __syncthreads();
        if (t < nr) {
            const uint64_t k = red[t];
            out_max[r0 + t] = key_value(k);
            out_idx[r0 + t] = key_index(k);
        }
        __syncthreads();
    }
}

// Host-side view of a workspace for n_rows output rows.
inline ArgmaxWs argmax_ws(void* workspace, int64_t n_rows) {
    ArgmaxWs w;
    w.keys = reinterpret_cast<unsigned long long*>(workspace);
    w.counters = reinterpret_cast<unsigned int*>(reinterpret_cast<char*>(workspace) + workspace_key_bytes(n_rows));
    w.P = workspace_partitions(n_rows);
    w.stride = workspace_key_stride(n_rows);
    return w;
}

}  // namespace mtpd
