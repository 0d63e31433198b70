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

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima).
#define MTPD_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Position of chunk c (16 bytes, 0..3) of row r's 64-byte K half inside the
// row's slot of a piece.  A fragment read has lane l on row l % 16 and K
// group l / 16; with the chunk moved to c ^ ((r >> 1) & 3) the hardware's
// bank-conflict counter reads zero for that read on gfx950 (an LDS probe of
// this exact pattern; c ^ ((r >> 1) ^ (r >> 3)) & 3, c ^ (r & 3) and no
// swizzle all counted conflicts).
__device__ __forceinline__ int piece_chunk(int r, int c) { return c ^ ((r >> 1) & 3); }

// Workgroup barrier without a memory fence: the LDS-DMA copies a wave must
// have finished are waited for explicitly (MTPD_WAIT_VMCNT) just before, and
// the memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

__global__ __launch_bounds__(512) void lmhead_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int n_row_tiles, int n_col_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx, ArgmaxWs ws)
{
    // two distinct objects, so LDS-DMA writes into one and fragment reads of
    // the other are independent to the compiler
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
    // global memory into LDS (no VGPRs); waves 0-3 also copy the 256 scales.
    // In one copy instruction lanes 4q..4q+3 read the four 16-byte chunks of
    // row q's K half (one 64-byte segment, so the address unit coalesces
    // them), in the swizzled order piece_chunk(q, .).  Per-lane addresses are
    // 32-bit byte offsets from wave-uniform bases (the host keeps the
    // activation under 4 GiB), so a K step only moves the scalar base.
    const int crow = lane >> 2;
    const uint32_t cchunk = (uint32_t)piece_chunk(crow, lane & 3) * 16u;
    uint32_t aoff[2], woff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = min(m0 + (2 * wave + i) * 16 + crow, n_rows - 1);
        const uint32_t a = (uint32_t)(row_index ? row_index[m] : m);
        aoff[i] = a * (uint32_t)H + cchunk;
        woff[i] = (uint32_t)((2 * wave + i) * 16 + crow) * (uint32_t)H + cchunk;
    }
    const uint8_t* wbase = w_codes + (size_t)n0 * (size_t)H;
    const int sa_row = min(m0 + (t & (kBM - 1)), n_rows - 1);
    const uint32_t saoff = (uint32_t)(row_index ? row_index[sa_row] : sa_row) * (uint32_t)KB;
    const float* swp = w_scales + (size_t)((n0 + wn * 64) >> 7) * KB;

    auto copy_in = [&](Stage& st, int kb) {
        const uint8_t* ab = a_codes + (size_t)kb * kBlock;
        const uint8_t* wb = wbase + (size_t)kb * kBlock;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                __builtin_amdgcn_global_load_lds(ab + aoff[i] + h * 64,
                                                 (lds_void_ptr)&st.piece[(4 * wave + 2 * i + h) * 64], 16, 0, 0);
                __builtin_amdgcn_global_load_lds(wb + woff[i] + h * 64,
                                                 (lds_void_ptr)&st.piece[(kPieces + 4 * wave + 2 * i + h) * 64], 16,
                                                 0, 0);
            }
        }
        if (wave < 4)
            __builtin_amdgcn_global_load_lds(a_scales + kb + saoff, (lds_void_ptr)&st.sa[wave * 64], 4, 0, 0);
    };
    // MFMA lane l takes row l % 16 and K group l / 16 of a piece: the uint4
    // holding that chunk
    const int frag = 4 * (lane & 15) + piece_chunk(lane & 15, lane >> 4);

    float acc[8][4][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

    // Per K block the wave runs 8 row groups of 4 MFMAs (one per column
    // tile).  The partials of group mt are folded into the accumulators
    // during group mt + 1, one column tile per MFMA, so every promotion FMA
    // reads a result four matrix instructions old and issues while the
    // matrix core works; the last group's promotion is carried into the next
    // block, where it covers the wait for that block's first fragments.
    v4f pr[2][4];
    float f[2][4];
    v8i af[2];
    float4 sav[2];
    v8i bf[4];

    auto load_a = [&](const Stage& st, int mt, int slot) {
        const uint4* As = &st.piece[0];
        const int p = (wm * 8 + mt) * 2;
        af[slot] = make_frag(As[p * 64 + frag], As[(p + 1) * 64 + frag]);
        sav[slot] = *reinterpret_cast<const float4*>(&st.sa[wm * 128 + mt * 16 + 4 * (lane >> 4)]);
    };
    auto promote = [&](int mt, int slot, int nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = fmaf(pr[slot][nt][r], f[slot][r], acc[mt][nt][r]);
    };

    // before the first block the carried partials are zero; the empty asm
    // hides the zero accumulators from constant folding, so the first block
    // compiles to the same FMAs as every other one
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) pr[1][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) f[1][r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(acc[i][j][r]));

    auto compute = [&](const Stage& st, int kb) {
        const float sw = scalar_load(swp, kb);
        const uint4* Ws = &st.piece[kPieces * 64];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int p = (wn * 4 + nt) * 2;
            bf[nt] = make_frag(Ws[p * 64 + frag], Ws[(p + 1) * 64 + frag]);
        }
        load_a(st, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) promote(7, 1, nt);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int slot = mt & 1;
            f[slot][0] = sav[slot].x * sw;
            f[slot][1] = sav[slot].y * sw;
            f[slot][2] = sav[slot].z * sw;
            f[slot][3] = sav[slot].w * sw;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                pr[slot][nt] = mfma_e4m3(af[slot], bf[nt]);
                if (mt > 0) promote(mt - 1, slot ^ 1, nt);
                if (nt == 0 && mt < 7) load_a(st, mt + 1, slot ^ 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Pipeline: block kb is read from one buffer while the copy of block
    // kb + 1 fills the other; before the barrier ending a block each wave
    // waits for its own copies.  No branch sits between a block's FMAs and the
    // next block (one would let the compiler sink the FMAs past it).
    copy_in(stage0, 0);
    MTPD_WAIT_VMCNT(0);
    bare_barrier();
    // K blocks in pairs so each half names its buffers at compile time
    for (int kb = 0; kb < KB; kb += 2) {
        if (kb + 1 < KB) copy_in(stage1, kb + 1);
        compute(stage0, kb);
        MTPD_WAIT_VMCNT(0);
        bare_barrier();
        if (kb + 1 < KB) {
            if (kb + 2 < KB) copy_in(stage0, kb + 2);
            compute(stage1, kb + 1);
            MTPD_WAIT_VMCNT(0);
            bare_barrier();
        }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) promote(7, 1, nt);

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
            best = row16_max_u64(best);
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
