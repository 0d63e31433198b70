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

#include <stdio.h>

#include <algorithm>

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


// ---------------------------------------------------------------------------
// Pipelined form: the same tile algebra with the LDS fragment reads issued
// from inline asm and their waits placed by hand.
//
//  - BM = 32 * MT activation rows x 256 vocab rows per workgroup (8 waves,
//    2 x 4, each 16 * MT rows x 64 columns).  MT = 8 gives 256-row tiles;
//    MT = 5 160-row tiles; MT = 10 320-row tiles (257 to 320 rows in one
//    tile, so each weight tile is copied once).  Row tiles go in groups of
//    `group_rows`, row fastest inside a group, consecutive ids on one XCD:
//    with groups of 8 (the 256-row tile's default) an XCD's 32 workgroups
//    cover 8 row x 4 column tiles.
//  - Staging: per K block both operand tiles go global -> LDS as [row][128
//    bytes], eight consecutive lanes per row's 128 bytes (a whole cache line
//    per eight lanes: measured 12.4 against 10.7 TB/s of L2 -> LDS for four
//    lanes per 64-byte half, copies alone, every CU busy), chunk c of row r
//    at position c ^ ((r >> 1) & 7).  Global loads with a wave-uniform base
//    and 32-bit lane offsets (buffer loads measured 5% slower); the next
//    block's copies are spread over the current block's MFMAs, one after
//    each from the fifth on.
//  - MFMA lane l supplies row l % 16 and, for its 32 K bytes, 16-byte chunks
//    l / 16 and l / 16 + 4 of that row (A and B permute K the same way, so
//    the dot product is unchanged): each of the two fragment reads then
//    touches 16 rows at one chunk each, and the swizzle spreads any 16
//    consecutive lanes over all 64 banks.
//  - Operand order: each MFMA takes the weight fragment first, so a lane's
//    four results of one MFMA are four vocab columns of one activation row.
//    They share one promotion factor, and the row's argmax is mostly in-lane
//    work: 16 values per lane and row group, then two cross-lane steps
//    (about 470 VALU instructions per wave for the epilogue, against about
//    860 with the activation fragment first; the FMAs and matrix
//    instructions together fill about 90% of the SIMD cycles, so every VALU
//    instruction costs time).  Measured on compute_stress in one call:
//    6.14 against 6.25 ms; mtp5_batch unchanged.
//  - Block scales: the activation scales arrive eight K blocks at a time
//    (32 bytes per row, two lanes per row: one request per eight rows'
//    lines instead of one per row per block, which cost 15% of the copy
//    rate); during block kb every thread forms one entry sa[row] * sw[block]
//    of block kb + 1's factor table (2 weight-scale blocks x BM rows), so
//    the promotion reads its factors instead of multiplying them per wave.
//    The table is in lane order, so a lane reads its MT factors of a block
//    in MT / 4 16-byte reads and one 8- or 4-byte read.
//  - Per K block a wave issues its first row group's activation fragment and
//    factors and its four weight fragments, then starts each of the first
//    group's MFMAs as soon as that MFMA's own operands have arrived (reads
//    return in issue order, so partial counts suffice); later groups wait
//    only for what the previous group issued.  The compiler's own waits
//    drained every read, the one just issued included.
// ---------------------------------------------------------------------------

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int MT>
struct G2 {
    static constexpr int BM = 32 * MT;                // activation rows per tile
    static constexpr int A_BYTES = BM * 128;          // activation tile, [row][128 bytes]
    static constexpr int W_BYTES = 256 * 128;         // weight tile
    // LDS, operand-major so that one base register per fragment half reaches
    // both stages through the 16-bit immediate offset: [A stage 0][A stage 1]
    // [W stage 0][W stage 1][scale chunk 0][scale chunk 1]
    static constexpr int W_OFF = 2 * A_BYTES;
    static constexpr int SC_OFF = W_OFF + 2 * W_BYTES;
    static constexpr int SC_BLOCKS = BM > 256 ? 4 : 8;   // K blocks per scale chunk (LDS budget)
    static constexpr int SC_BYTES = BM * SC_BLOCKS * 4;   // [row][SC_BLOCKS] fp32
    static constexpr int SC_LANES = SC_BLOCKS / 4;        // lanes per row of a chunk copy (16 bytes each)
    static constexpr int SMEM = SC_OFF + 2 * SC_BYTES;
    static constexpr int A_COPIES = BM / 8;           // copies of 8 rows x 128 bytes
    static constexpr int SCOPY = BM * SC_LANES / 64;  // scale-chunk copies (64 lanes x 16 bytes)
    static constexpr int SW_MAX = 64;                 // K blocks of the weight-scale table (H <= 8192)
    static_assert(MT <= 12, "row groups per wave (immediate-offset cases)");
};

// position of 16-byte chunk c of row r inside the row's 128 bytes
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int OFF>
__device__ __forceinline__ u32x4_t lds_read16_off(uint32_t addr) {
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// lds_read16_off<s * SBYTES + k * STEP>(addr) for a stage s (0, 1) and a k
// (0..11) known after unrolling
template <int SBYTES, int STEP>
__device__ __forceinline__ u32x4_t lds_read16_sk(uint32_t addr, int s, int k) {
    static_assert(SBYTES + 11 * STEP < 65536, "immediate offset range");
#define MTPD_CASE(S, K) \
    case S * 16 + K: return lds_read16_off<S * SBYTES + K * STEP>(addr);
#define MTPD_CASES(S)                                                                                     \
    MTPD_CASE(S, 0) MTPD_CASE(S, 1) MTPD_CASE(S, 2) MTPD_CASE(S, 3) MTPD_CASE(S, 4) MTPD_CASE(S, 5)      \
    MTPD_CASE(S, 6) MTPD_CASE(S, 7) MTPD_CASE(S, 8) MTPD_CASE(S, 9) MTPD_CASE(S, 10) MTPD_CASE(S, 11)
    switch (s * 16 + k) {
        MTPD_CASES(0)
        MTPD_CASES(1)
        default: __builtin_unreachable();
    }
#undef MTPD_CASES
#undef MTPD_CASE
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

template <int OFF>
__device__ __forceinline__ u32x2_t lds_read8_off(uint32_t addr) {
    u32x2_t v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_read4_off(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// The factor reads of stage s (0, 1): a full chunk c (0..2) of four row
// groups' factors, 16 bytes per lane; the partial chunk (one or two row
// groups) at stage offset only.  s and c are known after unrolling.
template <int SBYTES>
__device__ __forceinline__ u32x4_t lds_read_fchunk(uint32_t addr, int s, int c) {
    static_assert(SBYTES + 2 * 256 < 65536, "immediate offset range");
    switch (s * 4 + c) {
        case 0: return lds_read16_off<0>(addr);
        case 1: return lds_read16_off<256>(addr);
        case 2: return lds_read16_off<512>(addr);
        case 4: return lds_read16_off<SBYTES>(addr);
        case 5: return lds_read16_off<SBYTES + 256>(addr);
        case 6: return lds_read16_off<SBYTES + 512>(addr);
        default: __builtin_unreachable();
    }
}
template <int SBYTES>
__device__ __forceinline__ u32x2_t lds_read_fpart2(uint32_t addr, int s) {
    return s == 0 ? lds_read8_off<0>(addr) : lds_read8_off<SBYTES>(addr);
}
template <int SBYTES>
__device__ __forceinline__ uint32_t lds_read_fpart1(uint32_t addr, int s) {
    return s == 0 ? lds_read4_off<0>(addr) : lds_read4_off<SBYTES>(addr);
}

__device__ __forceinline__ v8i frag_of(u32x4_t lo, u32x4_t hi) {
    v8i f;
    f[0] = (int)lo[0]; f[1] = (int)lo[1]; f[2] = (int)lo[2]; f[3] = (int)lo[3];
    f[4] = (int)hi[0]; f[5] = (int)hi[1]; f[6] = (int)hi[2]; f[7] = (int)hi[3];
    return f;
}

// Waits until at most N LDS reads of this wave are outstanding (reads return
// in issue order); the registers those reads fill are tied to the wait, so no
// use of them is scheduled above it.  (Inline asm and device builtins live in
// device functions only: a kernel template whose own body holds them fails
// to instantiate in the host pass, and its launch stub is not emitted.)
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, u32x4_t& c) {
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, u32x4_t& c, u32x4_t& d) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, u32x4_t& c, u32x4_t& d, u32x4_t& e) {
    asm volatile("s_waitcnt lgkmcnt(%5)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, u32x2_t& c) {
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, uint32_t& c) {
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "n"(N));
}

// 1 if the predicate holds on any lane of the wave
__device__ __forceinline__ unsigned int any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0 ? 1u : 0u; }

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// scheduling fence: nothing moves across it
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// workgroup barrier after this wave's LDS accesses (the scale-table writes)
// and LDS-DMA copies have completed
__device__ __forceinline__ void drain_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// direct global -> LDS copies of 16 (4) bytes per lane, lane i's bytes to lds + i * 16 (4)
__device__ __forceinline__ void dma16(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 4, 0, 0);
}

// The same 16-byte copy from a wave-uniform base in SGPRs plus a 32-bit lane
// offset, written out so that no 64-bit lane address is formed (the builtin
// compiled to two 64-bit vector adds per copy inside the K loop).  M0 carries
// the LDS address (one wait state before the copy reads it).  The compiler
// neither sees nor waits for these copies: the kernel drains them itself
// (vmcnt(0) before each block's barrier).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; nothing else in the loop uses it
__device__ __forceinline__ void dma16_s(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// The same copy through a raw buffer resource of a given size: lanes whose
// byte offset lies past the end read zeros instead of faulting.  Third
// descriptor word: 32-bit data format, the raw-buffer setting of this
// architecture family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bdma16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// hides a value from constant folding (the zero accumulators of the first block)
__device__ __forceinline__ void opaque(float& x) { asm volatile("" : "+v"(x)); }

// the order-preserving u32 of a logit (argmax_key's upper word; -0 folds onto
// +0 through the addition)
__device__ __forceinline__ uint32_t ord_f32(float z) {
    const uint32_t u = __float_as_uint(z + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Per-row best of a wave's 16 x 64 sub-tiles, written to LDS.  The MFMAs
// take the weight fragment as their first operand, so lane l holds, for row
// group mt, the 16 values of activation row mt * 16 + l % 16 at columns
// col0 + 16 nt + 4 (l / 16) + r (nt, r = 0..3).  Each lane takes its largest
// value and the lowest of its columns holding it; the four lanes sharing a
// row (l, l + 16, l + 32, l + 48) then agree on the row's maximum and the
// lowest column among the lanes that hold it, and lane l < 16 writes the key
// to dst[mt * 16 + l].  fp32 compares treat -0 and +0 as equal, as the key
// does (ord_f32 folds -0 onto +0).
template <int MT>
__device__ __forceinline__ void row_best_keys(const float (&acc)[MT][4][4], int lane, uint32_t col0,
                                              unsigned long long* dst) {
    const uint32_t q4 = (uint32_t)(lane >> 4) * 4u;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float m = acc[mt][0][0];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[mt][nt][r]);
        uint32_t c = 0xFFFFu;
#pragma unroll
        for (int nt = 3; nt >= 0; --nt)
#pragma unroll
            for (int r = 3; r >= 0; --r) c = acc[mt][nt][r] == m ? (uint32_t)(nt * 16 + r) : c;
        c += q4;
        float mx = fmaxf(m, __shfl_xor(m, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        uint32_t cc = m == mx ? c : 0xFFFFu;
        cc = min(cc, (uint32_t)__shfl_xor((int)cc, 16));
        cc = min(cc, (uint32_t)__shfl_xor((int)cc, 32));
        if (lane < 16) dst[mt * 16 + lane] = ((uint64_t)ord_f32(mx) << 32) | (uint64_t)(0xFFFFFFFFu - (col0 + cc));
    }
}

}  // namespace

template <int MT>
__global__ __launch_bounds__(512) void lmhead_gemm2_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int n_row_tiles, int n_col_tiles, int group_rows, uint32_t scale_bytes,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx, ArgmaxWs ws)
{
    using C = G2<MT>;
    constexpr int BM = C::BM;
    static_assert(C::SMEM + 2 * 2 * BM * 4 + 2 * C::SW_MAX * 4 <= 160 * 1024, "LDS");
    static_assert(4 * BM * 8 <= C::SMEM, "epilogue table must fit in the stage memory");
    __shared__ __align__(16) unsigned char smem[C::SMEM];
    // promotion factors sa[row] * sw[block] of two K blocks (slots): per slot,
    // weight-scale block cb and row half wm, the 16 * MT factors of that half
    // in lane order: chunk c (row groups 4c .. 4c + 3) holds lane row j's four
    // at 16 j, the partial chunk (the last MT % 4 groups) its MT % 4 at
    // FP * 4 j, so a lane reads its factors for a block in MT / 4 16-byte reads
    // and one 8- or 4-byte read
    constexpr int FC = MT / 4, FP = MT % 4;
    static_assert(FC >= 1 && FC <= 3 && FP != 3, "factor chunks");
    __shared__ __align__(16) float ftab[2 * 2 * 2 * 16 * MT];
    __shared__ __align__(16) float swtab[2][C::SW_MAX];   // weight scales of the tile's two 128-row blocks
    __shared__ unsigned int deps[8];
    __shared__ int last_flag;

    const int KB = H >> 7;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = wave_uniform(t >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    // tile order: row tiles in groups of group_rows, row fastest inside a
    // group, then column; consecutive ids run together on one XCD
    const int total = n_row_tiles * n_col_tiles;
    const int id = xcd_contiguous((int)blockIdx.x, total);
    const int group_tiles = group_rows * n_col_tiles;
    const int grp = id / group_tiles;
    const int rows_in_grp = min(group_rows, n_row_tiles - grp * group_rows);
    const int in_grp = id - grp * group_tiles;
    const int rt = grp * group_rows + in_grp % rows_in_grp;
    const int ct = in_grp / rows_in_grp;
    const int m0 = rt * BM, n0 = ct * 256;

    // ---- copy assignment (global -> LDS, no VGPRs) ----
    // Copy j of an operand moves rows 8j .. 8j + 7: lane i lands at position
    // i & 7 of row 8j + (i >> 3), so it reads the chunk stored there.
    // Activation copies j = wave, wave + 8, ... (rows past n_rows repeat its
    // last row); weight copies 4 * wave .. 4 * wave + 3; scale-chunk copy
    // `wave` on the first SCOPY waves (rows 32w .. 32w + 31, lanes 2q, 2q + 1
    // the two halves of row q's 32 bytes; rows past n_rows repeat its last
    // row).  Offsets are 32-bit from wave-uniform bases (the host keeps the
    // activation under 2 GiB for this kernel).
    const int crow = lane >> 3;
    constexpr int AC = (C::A_COPIES + 7) / 8;
    uint32_t aoff[AC], woff[4];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int j = min(wave + 8 * i, C::A_COPIES - 1);
        const int r = j * 8 + crow;
        const int m = min(m0 + r, n_rows - 1);
        const uint32_t a = (uint32_t)(row_index ? row_index[m] : m);
        aoff[i] = a * (uint32_t)H + (uint32_t)chunk_pos(r, lane & 7) * 16u;   // chunk_pos is its own inverse in c
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (4 * wave + i) * 8 + crow;
        woff[i] = (uint32_t)r * (uint32_t)H + (uint32_t)chunk_pos(r, lane & 7) * 16u;
    }
    const uint8_t* wbase = w_codes + (size_t)n0 * (size_t)H;
    // the scale chunks through a buffer resource of the scales' exact size: a
    // last chunk that runs past a row's K blocks reads the next row's scales
    // (unused), or zeros past the end of the array, never unmapped memory
    const rsrc_t s_rs = make_rsrc(a_scales, scale_bytes);
    const int sc_row = min(m0 + min((wave * 64 + lane) / C::SC_LANES, BM - 1), n_rows - 1);
    const uint32_t scoff = (uint32_t)(row_index ? row_index[sc_row] : sc_row) * (uint32_t)KB * 4u +
                           (uint32_t)(lane % C::SC_LANES) * 16u;

    // codes of block kb into stage s
    auto copy_in = [&](int s, int kb) {
        const uint8_t* ab = a_codes + (size_t)kb * kBlock;
        const uint8_t* wb = wbase + (size_t)kb * kBlock;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int j = wave + 8 * i;
            if (j < C::A_COPIES) dma16(ab + aoff[i], smem + s * C::A_BYTES + j * 1024);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(wb + woff[i], smem + C::W_OFF + s * C::W_BYTES + (4 * wave + i) * 1024);
    };
    // Copy c (0 .. NCOPY - 1) of block kb into stage s: activation copies
    // first, then the four weight copies; the same copies as copy_in.
    constexpr int NCOPY = AC + 4;
    // The next block's copies go out one per MFMA, from the block's fifth
    // MFMA on: issued all at once at the block start they stalled every wave
    // at issue (the address unit takes a 1 KB copy per 16 clocks) before its
    // first fragment reads, and spread further apart they land too late
    // (measured on compute_stress: 6.9-7.1 ms at the block start, 6.5-6.6 ms
    // from the fifth MFMA, 6.7 ms at every second MFMA).
    // The 320-row tile (40 MFMAs per block, its weight copies from HBM) does
    // best with one copy after every second MFMA from the fifth on (mtp5_batch
    // 312-318 against 320-326 us, three interleaved rounds in one call; every
    // third MFMA 327-330 us, from the third or the ninth 315-324 us).
    constexpr int kCopyStart = 4;
    constexpr int kCopyStride = MT > 8 ? 2 : 1;
    static_assert(kCopyStart + kCopyStride * (NCOPY - 1) < 4 * MT, "every copy is issued inside the block");
    // copy number of MFMA n of the block, or -1
    auto copy_at = [](int n) {
        const int d = n - kCopyStart;
        return d >= 0 && d % kCopyStride == 0 && d / kCopyStride < NCOPY ? d / kCopyStride : -1;
    };
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    auto copy_one = [&](int s, int kb, int c) {
        if (c < AC) {
            const int j = wave + 8 * c;
            if (j < C::A_COPIES)
                dma16_s(a_codes + (size_t)kb * kBlock, aoff[c], smem_lds + (uint32_t)(s * C::A_BYTES + j * 1024));
        } else {
            const int i = c - AC;
            dma16_s(wbase + (size_t)kb * kBlock, woff[i],
                    smem_lds + (uint32_t)(C::W_OFF + s * C::W_BYTES + (4 * wave + i) * 1024));
        }
    };
    // activation scales of K blocks c * SC_BLOCKS .. + SC_BLOCKS - 1 into chunk slot c % 2
    auto copy_scales = [&](int c) {
        if (wave < C::SCOPY)
            bdma16(s_rs, scoff + (uint32_t)(c * C::SC_BLOCKS) * 4u, 0u,
                   smem + C::SC_OFF + (c & 1) * C::SC_BYTES + wave * 1024);
    };

    // ---- fragment addresses (bytes in LDS), one set per stage ----
    const int fr = lane & 15, fg = lane >> 4;
    const uint32_t lo16 = (uint32_t)(fr * 128 + chunk_pos(fr, fg) * 16);
    const uint32_t hi16 = (uint32_t)(fr * 128 + chunk_pos(fr, fg + 4) * 16);
    const uint32_t smem0 = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const uint32_t a_lo = smem0 + (uint32_t)(wm * MT * 16 * 128) + lo16;
    const uint32_t a_hi = smem0 + (uint32_t)(wm * MT * 16 * 128) + hi16;
    const uint32_t b_lo = smem0 + (uint32_t)(C::W_OFF + wn * 64 * 128) + lo16;
    const uint32_t b_hi = smem0 + (uint32_t)(C::W_OFF + wn * 64 * 128) + hi16;
    constexpr int FSLOT = 2 * 2 * 16 * MT * 4;   // bytes between the two factor slots
    const uint32_t f_reg = (uint32_t)(uintptr_t)(lds_ptr_t)&ftab[((wn >> 1) * 2 + wm) * 16 * MT];
    const uint32_t f_full = f_reg + (uint32_t)(fr * 16);
    const uint32_t f_part = f_reg + (uint32_t)(FC * 256 + fr * FP * 4);

    float acc[MT][4][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) opaque(acc[i][j][r]);

    v4f ring[3];        // the last three MFMA results, each folded in two MFMAs later

    // (each updated accumulator passes through an empty asm, so the FMA stays
    // where it is written: left alone, the compiler sinks every fold-in of a
    // block past the block's barrier, keeping all its MFMA results live).
    // The four values of a lane in one MFMA result share the lane's
    // activation row, so they share one factor.
    auto promote = [&](int mt, int nt, const v4f& p, uint32_t f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[mt][nt][r] = fmaf(p[r], __uint_as_float(f), acc[mt][nt][r]);
            opaque(acc[mt][nt][r]);
        }
    };

    // One K block from stage s, factor slot s.  MFMA n of the block (row
    // group n / 4, column group n % 4) takes the weight fragment as its first
    // operand and goes to ring[n % 3]; its fold-in follows MFMA n + 2: by then
    // the matrix result is ready without wait states (folding in one MFMA
    // later needed s_nop padding before every fold-in, and measured 2% slower
    // on both compute-regime workloads).
    // Reads: the block's first batch is row group 0's activation fragment, all
    // four weight fragments and the factors of row groups 0 .. 3 (after the
    // second weight fragment: the first fold-in follows the third MFMA), and
    // group 0's MFMAs start as their own operands arrive; group g + 1's
    // activation fragment (and, when g + 1 starts a chunk, that chunk of
    // factors) is issued after group g's first MFMA, into the activation slot
    // of group g - 1, whose MFMAs have all issued.
    auto compute = [&](int s, auto&& after) {
        u32x4_t alo[2], ahi[2], fc[FC];
        u32x2_t fp2 = {0u, 0u};
        uint32_t fp1 = 0u;
        alo[0] = lds_read16_sk<C::A_BYTES, 2048>(a_lo, s, 0);
        ahi[0] = lds_read16_sk<C::A_BYTES, 2048>(a_hi, s, 0);
        u32x4_t b0 = lds_read16_sk<C::W_BYTES, 2048>(b_lo, s, 0), b1 = lds_read16_sk<C::W_BYTES, 2048>(b_hi, s, 0);
        u32x4_t b2 = lds_read16_sk<C::W_BYTES, 2048>(b_lo, s, 1), b3 = lds_read16_sk<C::W_BYTES, 2048>(b_hi, s, 1);
        fc[0] = lds_read_fchunk<FSLOT>(f_full, s, 0);
        u32x4_t b4 = lds_read16_sk<C::W_BYTES, 2048>(b_lo, s, 2), b5 = lds_read16_sk<C::W_BYTES, 2048>(b_hi, s, 2);
        u32x4_t b6 = lds_read16_sk<C::W_BYTES, 2048>(b_lo, s, 3), b7 = lds_read16_sk<C::W_BYTES, 2048>(b_hi, s, 3);
        v8i bf[4];
        v8i af;
        auto factor = [&](int mt) -> uint32_t {
            if (mt < 4 * FC) return fc[mt >> 2][mt & 3];
            if constexpr (FP == 2) return fp2[mt - 4 * FC];
            return fp1;
        };
        // group 1's two reads follow group 0's first MFMA, so the waits for
        // weight fragments 1 .. 3 leave them (and the younger reads) in flight
        constexpr int NXT = MT > 1 ? 2 : 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int n = mt * 4 + nt;
                if (n == 0) {
                    // in flight: A0 (2), B0, B1 (4), F0, B2, B3 (4): the first 4 are group 0's and B0
                    lds_wait<7>(alo[0], ahi[0], b0, b1);
                    af = frag_of(alo[0], ahi[0]);
                    bf[0] = frag_of(b0, b1);
                } else if (n == 1) {
                    lds_wait<NXT + 5>(b2, b3);
                    bf[1] = frag_of(b2, b3);
                } else if (n == 2) {
                    lds_wait<NXT + 2>(b4, b5, fc[0]);
                    bf[2] = frag_of(b4, b5);
                } else if (n == 3) {
                    lds_wait<NXT>(b6, b7);
                    bf[3] = frag_of(b6, b7);
                } else if (nt == 0) {
                    if (mt % 4 == 0 && mt < 4 * FC) lds_wait<0>(alo[mt & 1], ahi[mt & 1], fc[mt >> 2]);
                    else if (mt == 4 * FC && FP == 2) lds_wait<0>(alo[mt & 1], ahi[mt & 1], fp2);
                    else if (mt == 4 * FC && FP == 1) lds_wait<0>(alo[mt & 1], ahi[mt & 1], fp1);
                    else lds_wait<0>(alo[mt & 1], ahi[mt & 1]);
                    af = frag_of(alo[mt & 1], ahi[mt & 1]);
                }
                sched_fence();
                ring[n % 3] = mfma_e4m3(bf[nt], af);
                sched_fence();
                after(n);
                sched_fence();   // the MFMA issues first, then an older one's fold-in
                if (n >= 2) promote((n - 2) >> 2, (n - 2) & 3, ring[(n - 2) % 3], factor((n - 2) >> 2));
                if (nt == 0 && mt + 1 < MT) {
                    alo[(mt + 1) & 1] = lds_read16_sk<C::A_BYTES, 2048>(a_lo, s, mt + 1);
                    ahi[(mt + 1) & 1] = lds_read16_sk<C::A_BYTES, 2048>(a_hi, s, mt + 1);
                    if ((mt + 1) % 4 == 0 && mt + 1 < 4 * FC) fc[(mt + 1) >> 2] = lds_read_fchunk<FSLOT>(f_full, s, (mt + 1) >> 2);
                    if (mt + 1 == 4 * FC) {
                        if constexpr (FP == 2) fp2 = lds_read_fpart2<FSLOT>(f_part, s);
                        if constexpr (FP == 1) fp1 = lds_read_fpart1<FSLOT>(f_part, s);
                    }
                }
                sched_fence();
            }
#pragma unroll
        for (int n = 4 * MT - 2; n < 4 * MT; ++n) promote(n >> 2, n & 3, ring[n % 3], factor(n >> 2));
    };

    // promotion factors of block kb from its scale chunk
    // (thread t: weight-scale block t / BM, row t % BM)
    // With one entry per thread (tiles of up to 256 rows) each thread reads its
    // row's scales of four blocks as one float4 on every fourth block and keeps
    // them in registers for the three blocks after: a row's blocks are
    // contiguous in the chunk, and one 4-byte read per block put the 64 rows a
    // wave reads on 8 banks.  The 320-row tile (two entries for some threads,
    // no registers to spare) reads one scale per block.
    float4 sa4 = make_float4(0.f, 0.f, 0.f, 0.f);
    // position in slot 0 of the factor of weight-scale block cb and tile row r
    auto fpos = [](int cb, int r) {
        const int wm_ = r / (16 * MT), rem = r - wm_ * 16 * MT, mt = rem >> 4, j = rem & 15;
        const int in = mt < 4 * FC ? 64 * (mt >> 2) + 4 * j + (mt & 3) : 64 * FC + FP * j + (mt - 4 * FC);
        return (cb * 2 + wm_) * 16 * MT + in;
    };
    constexpr int FSLOTF = FSLOT / 4;
    const int fpos_t = t < 2 * BM ? fpos(t / BM, t % BM) : 0;
    auto factors = [&](int slot, int kb) {
        const float* chunk =
            reinterpret_cast<const float*>(smem + C::SC_OFF + ((kb / C::SC_BLOCKS) & 1) * C::SC_BYTES);
        const int k = kb % C::SC_BLOCKS;
        if constexpr (2 * BM <= 512) {
            if (t < 2 * BM) {
                const int cb = t / BM, r = t - cb * BM;
                if ((k & 3) == 0) sa4 = *reinterpret_cast<const float4*>(&chunk[r * C::SC_BLOCKS + k]);
                const float sa = (k & 3) == 0 ? sa4.x : (k & 3) == 1 ? sa4.y : (k & 3) == 2 ? sa4.z : sa4.w;
                ftab[slot * FSLOTF + fpos_t] = sa * swtab[cb][kb];
            }
        } else {
            for (int e = t; e < 2 * BM; e += 512) {
                const int cb = e / BM, r = e - cb * BM;
                ftab[slot * FSLOTF + fpos(cb, r)] = chunk[r * C::SC_BLOCKS + k] * swtab[cb][kb];
            }
        }
    };

    // ---- pipeline ----
    // Prologue: the weight-scale table, scale chunks 0 and 1, stage 0 = codes
    // of block 0; then block 0's factors.  Block kb computes from stage kb % 2
    // and factor slot kb % 2, while the copy of block kb + 1 (issued from
    // inside the block's MFMA sequence) fills the other stage and every thread
    // forms one factor of block kb + 1; the barrier ending the block publishes
    // both.  Chunk c + 1 is copied at the start of
    // block 8c (c >= 1): chunk c - 1, in that slot, was last read during block
    // 8c - 2.
    if (wave < 2)
        dma4(w_scales + (size_t)((n0 >> 7) + wave) * KB + min(lane, KB - 1), &swtab[wave][0]);
    copy_scales(0);
    if (KB > C::SC_BLOCKS) copy_scales(1);
    copy_in(0, 0);
    drain_barrier();
    factors(0, 0);
    drain_barrier();
    for (int kb = 0; kb < KB; kb += 2) {
        // stage 0 (kb is even: chunk boundaries fall here)
        if (kb > 0 && kb % C::SC_BLOCKS == 0 && kb + C::SC_BLOCKS < KB) copy_scales(kb / C::SC_BLOCKS + 1);
        compute(0, [&](int n) {
            if (copy_at(n) >= 0 && kb + 1 < KB) copy_one(1, kb + 1, copy_at(n));
        });
        if (kb + 1 < KB) factors(1, kb + 1);
        drain_barrier();
        if (kb + 1 >= KB) break;
        // stage 1
        compute(1, [&](int n) {
            if (copy_at(n) >= 0 && kb + 2 < KB) copy_one(0, kb + 2, copy_at(n));
        });
        if (kb + 2 < KB) factors(0, kb + 2);
        drain_barrier();
    }

    // ---- epilogue: per-row best over the wave's 64 columns, then over the
    // four column waves (table in the now idle stage memory).  A row's best
    // is its largest fp32 value and the lowest column holding it (fp32
    // compares treat -0 and +0 as equal, as the key does): the 32-bit
    // reductions cost a third of reducing 64-bit keys. ----
    unsigned long long* red = reinterpret_cast<unsigned long long*>(smem);
    row_best_keys<MT>(acc, lane, (uint32_t)(n0 + wn * 64), red + wn * BM + wm * MT * 16);
    __syncthreads();
    uint64_t old = 0;
    if (t < BM && m0 + t < n_rows) {
        const uint64_t k = u64_max(u64_max(red[t], red[BM + t]), u64_max(red[2 * BM + t], red[3 * BM + t]));
        old = merge_key(ws, n_rows, id, m0 + t, k);
    }
    const unsigned int dep = any_lane(never_nonzero(old) != 0);
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

template <int MT>
hipError_t launch_gemm2(const LmheadArgs& a, int group_rows, hipStream_t stream) {
    constexpr int BM = 32 * MT;
    const int64_t row_tiles = (a.n_rows + BM - 1) / BM;
    const int64_t col_tiles = a.V / 256;
    if (row_tiles * col_tiles > 0x7FFFFFFF || a.H > 128 * G2<MT>::SW_MAX || a.a_rows * a.H >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    const int gr = (int)std::max<int64_t>(1, std::min<int64_t>(group_rows, row_tiles));
    hipLaunchKernelGGL((lmhead_gemm2_kernel<MT>), dim3((unsigned)(row_tiles * col_tiles)), dim3(512), 0, stream,
                       a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales, (int)a.H,
                       (int)row_tiles, (int)col_tiles, gr, (uint32_t)(a.a_rows * (a.H / 128) * 4), a.out_max,
                       a.out_idx, argmax_ws(a.workspace, a.n_rows));
    return hipGetLastError();
}

int gemm_variant(int64_t n_rows, int64_t H, int64_t a_rows) {
    const int o = plan_override().gemm;
    if (o >= 1 && o <= 8) return o;
    // the pipelined kernel takes H <= 8192 (its weight-scale table) and an
    // activation under 2 GiB (32-bit buffer offsets)
    if (H > 128 * G2<8>::SW_MAX || a_rows * H >= ((int64_t)1 << 31)) return 1;
    // tile height: fewest copied bytes, row tiles x (tile rows + 256 weight
    // rows) per K block; the 320-row tile (its LDS full, scale chunks of four
    // blocks, every register in use) measured about 10% slower per byte, so
    // it is charged 10% more.  320 rows: one 320-row tile (each weight tile
    // copied once), not two 256-row tiles of which 192 rows are padding.
    const int64_t c8 = (n_rows + 255) / 256 * (256 + 256) * 10, c5 = (n_rows + 159) / 160 * (160 + 256) * 10;
    const int64_t c10 = (n_rows + 319) / 320 * (320 + 256) * 11;
    if (c10 < c8 && c10 < c5) return 8;
    // 256-row tiles in groups of 8 row tiles (an XCD's 32 workgroups then
    // cover 8 row x 4 column tiles): measured on compute_stress with the
    // weight fragment as the first MFMA operand, groups of 4, 8 and 16 took
    // 6.37-6.40, 6.32-6.36 and 6.44-6.45 ms (eight interleaved pairs of 4
    // and 8 in two calls, 8 faster in every pair); with the activation
    // fragment first, groups of 1, 2, 4, 8 and 16 had taken 7.09, 6.74-6.78,
    // 6.56-6.62, 6.62-6.65 and 6.73 ms
    return c5 < c8 ? 6 : 3;
}

void describe_gemm(int64_t n_rows, int64_t V, int64_t H, int64_t a_rows, char* buf, size_t len) {
    const int v = gemm_variant(n_rows, H, a_rows);
    const int bm = v == 1 ? 256 : (v <= 4 ? 256 : (v <= 6 ? 160 : 320));
    const long long tiles = (long long)((n_rows + bm - 1) / bm * (V / 256));
    if (v == 1) snprintf(buf, len, "lmhead_gemm_kernel grid=%lldx512", tiles);
    else snprintf(buf, len, "lmhead_gemm2_kernel<%d> grid=%lldx512 group=%d", bm / 32, tiles,
                  v == 2 || v == 5 || v == 7 ? 4 : (v == 4 ? 16 : 8));
}

hipError_t launch_lmhead_gemm(const LmheadArgs& a, hipStream_t stream) {
    // variant 1: the single-wait kernel; 2..6: pipelined shapes
    switch (gemm_variant(a.n_rows, a.H, a.a_rows)) {
        case 2: return launch_gemm2<8>(a, 4, stream);
        case 3: return launch_gemm2<8>(a, 8, stream);
        case 4: return launch_gemm2<8>(a, 16, stream);
        case 5: return launch_gemm2<5>(a, 4, stream);
        case 6: return launch_gemm2<5>(a, 8, stream);
        case 7: return launch_gemm2<10>(a, 4, stream);
        case 8: return launch_gemm2<10>(a, 8, stream);
        default: break;
    }
    const int64_t row_tiles = (a.n_rows + kBM - 1) / kBM;
    const int64_t col_tiles = a.V / kBN;
    if (row_tiles * col_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lmhead_gemm_kernel, dim3((unsigned)(row_tiles * col_tiles)), dim3(512), 0, stream,
                       a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales, (int)a.H,
                       (int)row_tiles, (int)col_tiles, a.out_max, a.out_idx, argmax_ws(a.workspace, a.n_rows));
    return hipGetLastError();
}

}  // namespace mtpd
