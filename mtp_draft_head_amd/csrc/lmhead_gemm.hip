// Block-scaled FP8 LM head + greedy argmax for many activation rows (the
// compute-bound regime): a 256 x 256 output tile per workgroup, both operands
// staged through LDS.
//
// Result definition as in lmhead_argmax.hip ("[Quant][MTP] Reuse packed FP8
// logits inputs", Purpose and Dependencies; "[Spec Decode][Perf] Fuse the MTP
// trailing all-reduce; local-argmax draft tokens", Summary).  Schedule:
//
//  - Workgroup = 8 waves in a 2 x 4 grid, each wave a 128 x 64 sub-tile:
//    8 x 4 MFMA 16x16x128 tiles, i.e. 32 matrix instructions per 128-wide K
//    scale block, each giving an unscaled block partial that the wave folds
//    into its fp32 accumulators as acc += p * (sa[row] * sw) (128 VALU FMAs
//    per 32 MFMAs, issued while the matrix core works on later tiles).  The
//    128 fp32 accumulators must live in VGPRs (the promotion is VALU work),
//    which is what bounds the wave tile: two waves per SIMD, 256 registers each.
//  - Per K block the workgroup stages the activation tile (256 rows x 128 B),
//    the weight tile (256 rows x 128 B) and the 256 activation scales of that
//    block into one of two LDS buffers with direct global-to-LDS loads (no
//    VGPRs; the accumulators need them).  The next block's copy is issued
//    before the current block's MFMAs; the barrier ending the block waits for
//    it.
//  - LDS holds fragments in MFMA order: a 1 KB piece per (16-row tile, K
//    half) with lane l's 16 bytes at l*16, so every fragment read is one
//    conflict-free 16-byte LDS load per lane.
//  - Tiles are ordered so each XCD's 32 concurrently running workgroups
//    cover 4 activation row tiles x 8 weight column tiles (operands shared
//    through that XCD's L2), and a weight column tile is fetched from HBM
//    once per 4 row tiles.
//  - Epilogue: per-row best keys of the two column waves meet in LDS, one
//    merge per row into the partitioned key slots, arrival, and the last
//    workgroup decodes (lmhead_common.h).

#include "kernels.h"
#include "lmhead_common.h"

namespace mtpd {

namespace {

constexpr int kBM = 256;                 // activation rows per tile
constexpr int kBN = 256;                 // vocab rows per tile
constexpr int kPieces = kBM / 16 * 2;    // 1 KB fragment pieces per operand per K block (32)
constexpr int kGroupRows = 4;            // row tiles per L2 super-group

}  // namespace

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// One K block's tiles in LDS, in MFMA fragment order: pieces [0, 32) are the
// activation's (16-row tile, K half), pieces [32, 64) the weight's; each piece
// is 64 lanes x 16 bytes.  sa: the 256 activation scales of the block.
struct Stage {
    uint4 piece[2 * kPieces * 64];
    float sa[kBM];
};

__global__ __launch_bounds__(512) void lmhead_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int n_row_tiles, int n_col_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx, ArgmaxWs ws)
{
    // two distinct objects, so the compiler can tell an LDS-DMA write into one
    // from fragment reads of the other and need not drain the DMA before them
    __shared__ __align__(16) Stage stage0;
    __shared__ __align__(16) Stage stage1;
    __shared__ unsigned long long red[4 * kBM];
    __shared__ unsigned int deps[8];
    __shared__ int last_flag;

    const int KB = H >> 7;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform, in an SGPR
    const int wm = wave >> 2, wn = wave & 3;    // 2 x 4 wave grid: 128 rows x 64 columns each

    // tile order: row tiles in groups of kGroupRows, row fastest inside a
    // group, then column; consecutive ids run together on one XCD
    const int total = n_row_tiles * n_col_tiles;
    const int id = xcd_contiguous((int)blockIdx.x, total);
    const int group_tiles = kGroupRows * n_col_tiles;
    const int grp = id / group_tiles;
    const int rows_in_grp = min(kGroupRows, n_row_tiles - grp * kGroupRows);
    const int in_grp = id - grp * group_tiles;
    const int rt = grp * kGroupRows + in_grp % rows_in_grp;
    const int ct = in_grp / rows_in_grp;
    const int m0 = rt * kBM, n0 = ct * kBN;

    // staging assignment: wave w copies A pieces and W pieces 4w..4w+3, i.e.
    // 16-row tiles 2w and 2w+1 of each operand, both K halves, straight from
    // global memory into LDS (no VGPRs); waves 0-3 also copy the 256 scales
    const uint8_t* ap[2];
    const uint8_t* wp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = min(m0 + (2 * wave + i) * 16 + (lane & 15), n_rows - 1);
        const int a = row_index ? row_index[m] : m;
        ap[i] = a_codes + (size_t)a * H + (lane >> 4) * 16;
        wp[i] = w_codes + (size_t)(n0 + (2 * wave + i) * 16 + (lane & 15)) * H + (lane >> 4) * 16;
    }
    const int sa_row = min(m0 + (t & (kBM - 1)), n_rows - 1);
    const float* sap = a_scales + (size_t)(row_index ? row_index[sa_row] : sa_row) * KB;
    const float* swp = w_scales + (size_t)((n0 + wn * 64) >> 7) * KB;

    auto copy_in = [&](Stage& st, int kb) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                __builtin_amdgcn_global_load_lds(ap[i] + kb * kBlock + h * 64,
                                                 (lds_void_ptr)&st.piece[(4 * wave + 2 * i + h) * 64], 16, 0, 0);
                __builtin_amdgcn_global_load_lds(wp[i] + kb * kBlock + h * 64,
                                                 (lds_void_ptr)&st.piece[(kPieces + 4 * wave + 2 * i + h) * 64], 16,
                                                 0, 0);
            }
        }
        if (wave < 4) __builtin_amdgcn_global_load_lds(sap + kb, (lds_void_ptr)&st.sa[wave * 64], 4, 0, 0);
    };

    float acc[8][4][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

    auto compute = [&](const Stage& st, int kb) {
        const float sw = scalar_load(swp, kb);
        const uint4* As = &st.piece[0];
        const uint4* Ws = &st.piece[kPieces * 64];
        v8i bf[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int p = (wn * 4 + nt) * 2;
            bf[nt] = make_frag(Ws[p * 64 + lane], Ws[(p + 1) * 64 + lane]);
        }
        // software pipeline over the 8 row tiles: the MFMAs of row tile mt are
        // issued before the promotion FMAs of row tile mt-1, so the matrix core
        // and the VALU overlap while only two groups of partials are live
        v4f pr[2][4];
        float f[2][4];
        auto mma = [&](int mt, int slot) {
            const int p = (wm * 8 + mt) * 2;
            const v8i af = make_frag(As[p * 64 + lane], As[(p + 1) * 64 + lane]);
            const float4 sa = *reinterpret_cast<const float4*>(&st.sa[wm * 128 + mt * 16 + 4 * (lane >> 4)]);
            f[slot][0] = sa.x * sw;
            f[slot][1] = sa.y * sw;
            f[slot][2] = sa.z * sw;
            f[slot][3] = sa.w * sw;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) pr[slot][nt] = mfma_e4m3(af, bf[nt]);
        };
        auto promote = [&](int mt, int slot) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][nt][r] = fmaf(pr[slot][nt][r], f[slot][r], acc[mt][nt][r]);
        };
        mma(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 1; mt < 8; ++mt) {
            mma(mt, mt & 1);
            promote(mt - 1, (mt - 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        promote(7, 1);
    };

    copy_in(stage0, 0);
    __syncthreads();
    // K blocks in pairs so each half names its buffers at compile time; the
    // copy of the next block is issued before the current block's MFMAs and
    // the barrier that ends the block waits for it
    for (int kb = 0; kb < KB; kb += 2) {
        if (kb + 1 < KB) copy_in(stage1, kb + 1);
        compute(stage0, kb);
        __syncthreads();
        if (kb + 1 < KB) {
            if (kb + 2 < KB) copy_in(stage0, kb + 2);
            compute(stage1, kb + 1);
            __syncthreads();
        }
    }

    // per-row best over this wave's 64 columns, then over the four column waves
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint64_t best = 0;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                best = u64_max(best, argmax_key(acc[mt][nt][i],
                                                (uint32_t)(n0 + wn * 64 + nt * 16 + (lane & 15))));
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) best = u64_max(best, shfl_xor_u64(best, off));
            if ((lane & 15) == 0) red[wn * kBM + wm * 128 + mt * 16 + 4 * (lane >> 4) + i] = best;
        }
    }
    __syncthreads();
    uint64_t old = 0;
    if (t < kBM && m0 + t < n_rows) {
        const uint64_t k = u64_max(u64_max(red[t], red[kBM + t]), u64_max(red[2 * kBM + t], red[3 * kBM + t]));
        old = merge_key(ws, n_rows, id, m0 + t, k);
    }
    // each wave waits for its own merges to return before the barrier, so the
    // arrival below follows every merge of this workgroup
    const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
    if (lane == 0) deps[wave] = dep;
    __syncthreads();
    if (t == 0) {
        unsigned int d = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) d |= deps[w];
        last_flag = arrive(ws, id, total, d) ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<512>(ws, n_rows, out_max, out_idx, red);
}

hipError_t launch_lmhead_gemm(const LmheadArgs& a, hipStream_t stream) {
    const int64_t row_tiles = (a.n_rows + kBM - 1) / kBM;
    const int64_t col_tiles = a.V / kBN;
    if (row_tiles * col_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lmhead_gemm_kernel, dim3((unsigned)(row_tiles * col_tiles)), dim3(512), 0, stream,
                       a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales, (int)a.H,
                       (int)row_tiles, (int)col_tiles, a.out_max, a.out_idx, argmax_ws(a.workspace, a.n_rows));
    return hipGetLastError();
}

}  // namespace mtpd
