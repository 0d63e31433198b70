// Vocab-parallel combines of local LM-head results for gfx950: greedy
// argmaxes, and below, top-k lists.
//
// Under vocab parallelism each GPU's LM head covers one contiguous slice of
// the vocabulary and returns a local (max logit, index) pair per row, so the
// full-vocab logits are never gathered ("[Spec Decode][Perf] Fuse the MTP
// trailing all-reduce; local-argmax draft tokens", Summary).  The global
// draft token is the pair with the largest max; among equal maxima the
// lowest global index wins, which is what a single full-vocab argmax with
// the lowest-index rule returns.  Each pair is packed into the same 64-bit
// key the LM-head epilogue uses (order-preserving logit bits above, the
// complement of the global index below), so the combine is a u64 maximum --
// the reduction a u64 MAX all-reduce performs across GPUs.
//
// One thread per row; shard s's pairs are read as one coalesced row of
// [n_shards][n_rows].  Bytes: 8 per pair read, 8 per row written.

#include "device_common.h"
#include "kernels.h"

namespace mtpd {

__global__ __launch_bounds__(256) void argmax_combine_kernel(
    const float* __restrict__ local_max, const int32_t* __restrict__ local_idx, ShardOffsets offs,
    int n_shards, int n_rows, float* __restrict__ out_max, int32_t* __restrict__ out_idx)
{
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= n_rows) return;
    uint64_t best = 0;
    for (int s = 0; s < n_shards; ++s) {
        const size_t e = (size_t)s * (size_t)n_rows + (size_t)r;
        best = u64_max(best, argmax_key(local_max[e], offs.off[s] + (uint32_t)local_idx[e]));
    }
    out_max[r] = key_value(best);
    out_idx[r] = key_index(best);
}

hipError_t launch_argmax_combine(const float* local_max, const int32_t* local_idx, const ShardOffsets& offs,
                                 int n_shards, int64_t n_rows, float* out_max, int32_t* out_idx,
                                 hipStream_t stream)
{
    if (n_shards < 1 || n_shards > kMaxShards || n_rows < 1 || n_rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((n_rows + 255) / 256);
    hipLaunchKernelGGL(argmax_combine_kernel, dim3(blocks), dim3(256), 0, stream, local_max, local_idx, offs,
                       n_shards, (int)n_rows, out_max, out_idx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The same combine for local top-k lists: shard s returns, per row, its k
// largest logits in descending order with local indices
// (mtpd_fp8_lmhead_topk), and the global top-k is selected from those lists
// instead of from gathered logits (same passages; the top-8 and top-32 sets
// are what "feat(glm52): add checkpoint-native MTP speculative decoding",
// Accuracy, compares).  Each pair becomes the epilogue's 64-bit key around
// its global index, so "largest value, then lowest index" is a u64 maximum
// and keys are distinct across shards.
//
// One wavefront per row (four rows per 256-thread workgroup): lane s holds
// the head of shard s's list (its k keys staged in LDS, column s), and each
// of k rounds takes the wave's largest head, which exactly one lane holds;
// that lane moves to its next key.  Lanes past n_shards hold key 0, below
// every real key.  Bytes: 8 per candidate read, 8 per output written.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = row16_max_u64(v);
    uint64_t m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * q);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * q);
        m = u64_max(m, ((uint64_t)hi << 32) | lo);
    }
    return m;
}

__global__ __launch_bounds__(256) void topk_combine_kernel(
    const float* __restrict__ local_val, const int32_t* __restrict__ local_idx, ShardOffsets offs,
    int n_shards, int n_rows, int k, float* __restrict__ out_val, int32_t* __restrict__ out_idx)
{
    __shared__ unsigned long long lists[4][kMaxTopk][64];   // [wave][list position][shard]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = (int)blockIdx.x * 4 + w;
    if (r >= n_rows) return;   // the whole wave; nothing below synchronizes across waves
    const bool live = lane < n_shards;
    if (live) {
        const size_t base = ((size_t)lane * (size_t)n_rows + (size_t)r) * (size_t)k;
        for (int j = 0; j < k; ++j)
            lists[w][j][lane] = argmax_key(local_val[base + j], offs.off[lane] + (uint32_t)local_idx[base + j]);
    }
    // each lane reads back only what it wrote itself
    int head = 0;
    uint64_t cur = live ? lists[w][0][lane] : 0;
    for (int e = 0; e < k; ++e) {
        const uint64_t m = wave_max_u64(cur);
        if (lane == 0) {
            out_val[(size_t)r * k + e] = key_value(m);
            out_idx[(size_t)r * k + e] = key_index(m);
        }
        if (live && cur == m) {
            ++head;
            cur = head < k ? lists[w][head][lane] : 0;
        }
    }
}

hipError_t launch_topk_combine(const float* local_val, const int32_t* local_idx, const ShardOffsets& offs,
                               int n_shards, int64_t n_rows, int k, float* out_val, int32_t* out_idx,
                               hipStream_t stream)
{
    if (n_shards < 1 || n_shards > kMaxShards || n_rows < 1 || n_rows > 0x7FFFFFFF || k < 1 || k > kMaxTopk)
        return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((n_rows + 3) / 4);
    hipLaunchKernelGGL(topk_combine_kernel, dim3(blocks), dim3(256), 0, stream, local_val, local_idx, offs, n_shards,
                       (int)n_rows, k, out_val, out_idx);
    return hipGetLastError();
}

}  // namespace mtpd
