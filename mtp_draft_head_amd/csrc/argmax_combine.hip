// Vocab-parallel combine of greedy local argmaxes for gfx950.
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

}  // namespace mtpd
