// Block-scaled FP8 LM head + greedy argmax for at most 16 activation rows
// (one MFMA row tile): the weight is streamed once through a per-wave LDS
// ring and every other cost is small next to it.
//
// Result definition as in lmhead_argmax.hip ("[Quant][MTP] Reuse packed FP8
// logits inputs", Purpose and Dependencies; "[Spec Decode][Perf] Fuse the MTP
// trailing all-reduce; local-argmax draft tokens", Summary).  Schedule:
//
//  - A workgroup is one wave and owns NT 16-row weight tiles over the whole
//    K range, so waves never wait for each other before the epilogue.
//  - Weight blocks go global -> LDS with direct copies (no VGPRs), D blocks
//    ahead of the MFMAs.  In one copy instruction eight consecutive lanes
//    read one weight row's 128-byte block, so the address unit coalesces
//    them into full lines; the MFMA operand layout (lane l = row l % 16,
//    K group l / 16) would instead issue one request per lane, which caps
//    a CU well below its share of HBM bandwidth.  Inside a row's 128-byte
//    slot chunk c sits at position c ^ s(r); s makes the fragment reads
//    conflict-free (see ring_pos).  The weight copies are non-temporal
//    (read once per launch); measured 4-10% faster than default caching.
//  - The activation rows of a block (at most 8 * MA of them) travel in the
//    same ring slot the same way, so the loop has no vector-memory load into
//    registers at all: a register load would make the compiler drain the
//    whole ring at the loop head.  Fragment rows past the last activation
//    row read the last row again.  The activation scales of the 16 fragment
//    rows and the tiles' weight-scale row are copied into LDS the same way
//    before the ring starts, and each block's factors sa * sw are formed on
//    the fly.
//  - The vector-memory counter is in order, so waiting for block kb is a
//    fixed count of younger requests: every refill issues the same number
//    of instructions (the block index is clamped near the end, never
//    skipped), and the last D blocks are consumed with decreasing counts.
//  - Epilogue: the 16-lane shuffle max per activation row, one merge per row
//    into the partitioned key slots, arrival, and the last workgroup decodes
//    (lmhead_common.h).

#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "kernels.h"
#include "lmhead_common.h"

namespace mtpd {

namespace {

// vmcnt-only wait (gfx9 encoding, other counters at their maxima)
#define MTPD_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// The same with a count that is a constant only after unrolling (0..63).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
#define MTPD_W4(b) case b: MTPD_WAIT_VM(b); break; case b + 1: MTPD_WAIT_VM(b + 1); break; \
                   case b + 2: MTPD_WAIT_VM(b + 2); break; case b + 3: MTPD_WAIT_VM(b + 3); break;
        MTPD_W4(0) MTPD_W4(4) MTPD_W4(8) MTPD_W4(12) MTPD_W4(16) MTPD_W4(20) MTPD_W4(24) MTPD_W4(28)
        MTPD_W4(32) MTPD_W4(36) MTPD_W4(40) MTPD_W4(44) MTPD_W4(48) MTPD_W4(52) MTPD_W4(56) MTPD_W4(60)
#undef MTPD_W4
        default: MTPD_WAIT_VM(0); break;
    }
}

// Position of 16-byte chunk c (0..7) of tile row r inside the row's 128-byte
// LDS slot.  A fragment read has lane l on row l % 16 and K group l / 16;
// with the chunk moved to c ^ (r & 7) the hardware's bank-conflict counter
// reads zero for that read on gfx950 (an LDS probe of this exact pattern:
// the earlier c ^ ((r ^ (r >> 3)) & 7) counted 4 conflict cycles per read,
// no swizzle 12).
__device__ __forceinline__ int ring_pos(int r, int c) { return c ^ (r & 7); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 32-bit LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)(lds_ptr_t)p; }

// Direct global -> LDS copy of 16 bytes per lane (lane l lands at lds + 16 l)
// from sbase + voff.  Issued from inline asm, so the compiler's wait
// insertion neither sees nor waits for it: the kernel tracks these copies
// with its own vector-memory counts.  M0 carries the LDS address (one wait
// state before the copy reads it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; the kernel uses it for nothing else
__device__ __forceinline__ void lds_copy16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
// The same for the weight stream, marked non-temporal: each weight byte is
// read once per launch, so its lines should not push the activation blocks
// and scale tables (re-read by every workgroup) out of the caches.
__device__ __forceinline__ void lds_copy16_stream(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
// The same with 4 bytes per lane (lane l lands at lds + 4 l).
__device__ __forceinline__ void lds_copy4(const float* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int kStreamMaxH = 8192;
constexpr int kStreamMaxKB = kStreamMaxH / 128;   // one 64-lane copy holds a row's scales

}  // namespace

template <int NT, int MA, int D>
__global__ __launch_bounds__(64) void lmhead_stream_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int total_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx,
    ArgmaxWs ws)
{
    // ring slot (uint4s): NT weight tiles of 2 eight-row 1 KB pieces, then MA
    // activation pieces of 8 rows
    constexpr int SLOT = (NT * 2 + MA) * 64;
    constexpr int PER_BLOCK = NT * 2 + MA;   // vector-memory instructions per refill
    static_assert((D - 1) * PER_BLOCK <= 63, "vmcnt holds at most 63");
    __shared__ __align__(16) uint4 ring[D * SLOT];
    __shared__ unsigned long long red[64];
    __shared__ int last_flag;
    // scales, copied once: sa_lds[kb][r] for fragment row r (rows past the
    // last activation row repeat it; block-major, so a lane's four rows of a
    // block are one 16-byte read and the four lane groups hit distinct
    // banks), sw_lds[kb] for the tiles' 128-row block; entries past KB repeat
    // the last block
    __shared__ __align__(16) float sa_lds[kStreamMaxKB * 16];
    __shared__ __align__(16) float sw_lds[kStreamMaxKB];

    const int lane = threadIdx.x;
    const int KB = H >> 7;
    const int KBp = (KB + D - 1) / D * D;
    const int tile = xcd_contiguous((int)blockIdx.x, total_tiles);
    const int n0 = tile * (NT * 16);

    // activation copy: piece q, lane l reads chunk ring_pos(r, l % 8) of
    // activation row r = 8q + l / 8, clamped to the last row (slots past the
    // last row hold copies of it)
    uint32_t aoff[MA];
#pragma unroll
    for (int q = 0; q < MA; ++q) {
        const int r = 8 * q + (lane >> 3);
        const int mr = min(r, n_rows - 1);
        aoff[q] = (uint32_t)(row_index ? row_index[mr] : mr) * (uint32_t)H + (uint32_t)ring_pos(r, lane & 7) * 16u;
    }
    // weight copy offsets: piece q of tile nt covers rows 8q..8q+7; lane l
    // reads chunk ring_pos(row, l % 8) of row 8q + l / 8
    const uint8_t* wbase = w_codes + (size_t)n0 * (size_t)H;
    uint32_t woff[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int r = 8 * q + (lane >> 3);
            woff[nt][q] = (uint32_t)(nt * 16 + r) * (uint32_t)H + (uint32_t)ring_pos(r, lane & 7) * 16u;
        }
    // fragment read positions (uint4 index inside a tile's 2 KB): row r, K
    // group g takes chunks g and g + 4
    const int fr = lane & 15, fg = lane >> 4;
    const int fpos0 = fr * 8 + ring_pos(fr, fg);
    const int fpos1 = fr * 8 + ring_pos(fr, fg + 4);
    // activation fragment: rows 8*MA.. (MA = 1) fold onto rows 0..7
    const int ar = fr & (8 * MA - 1);
    const int apos0 = ar * 8 + ring_pos(ar, fg);
    const int apos1 = ar * 8 + ring_pos(ar, fg + 4);

    const uint32_t ring0 = lds_addr(ring);
    auto refill = [&](int j, int kb) {
        const uint8_t* wb = wbase + (size_t)kb * kBlock;
        const uint8_t* ab = a_codes + (size_t)kb * kBlock;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 2; ++q) lds_copy16_stream(wb, woff[nt][q], ring0 + (uint32_t)(j * SLOT + (nt * 2 + q) * 64) * 16u);
#pragma unroll
        for (int q = 0; q < MA; ++q) lds_copy16(ab, aoff[q], ring0 + (uint32_t)(j * SLOT + (NT * 2 + q) * 64) * 16u);
    };

    float acc[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] = 0.f;

    // scale reads: rows 4 * fg + i of block kb; padding blocks (kb >= KB) get
    // a zero factor.  Each block's partials are promoted one block late (pp,
    // pf), so the FMAs never wait for the MFMA just issued; the order of the
    // sum is unchanged.
    v4f pp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pp[nt] = v4f{0.f, 0.f, 0.f, 0.f};
    float4 pf = make_float4(0.f, 0.f, 0.f, 0.f);
    auto promote = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            acc[nt][0] = fmaf(pp[nt][0], pf.x, acc[nt][0]);
            acc[nt][1] = fmaf(pp[nt][1], pf.y, acc[nt][1]);
            acc[nt][2] = fmaf(pp[nt][2], pf.z, acc[nt][2]);
            acc[nt][3] = fmaf(pp[nt][3], pf.w, acc[nt][3]);
        }
    };
    auto compute = [&](int j, int kb) {
        const int kc = min(kb, kStreamMaxKB - 1);
        const float swl = sw_lds[kc];
        const float sw = kb < KB ? swl : 0.f;
        const float4 sa4 = *reinterpret_cast<const float4*>(&sa_lds[kc * 16 + 4 * fg]);
        const float4 f = make_float4(sa4.x * sw, sa4.y * sw, sa4.z * sw, sa4.w * sw);
        const uint4* ta = &ring[j * SLOT + NT * 128];
        const v8i af = make_frag(ta[apos0], ta[apos1]);
        v4f p[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint4* tw = &ring[j * SLOT + nt * 128];
            p[nt] = mfma_e4m3(af, make_frag(tw[fpos0], tw[fpos1]));
        }
        promote();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pp[nt] = p[nt];
        pf = f;
    };

    // prologue: the activation scales of the 16 fragment rows, loaded into
    // registers and stored block-major (register loads, all completed here,
    // before the first ring copy is issued: a register load completing after
    // the copies were issued would make the compiler wait for those too);
    // then the weight-scale row and the first D ring blocks, copies into LDS
    // older than any ring block, so the first ring wait covers them
    {
        const int r = lane & 15;
        const int mr = min(r, n_rows - 1);
        const uint32_t srow = (uint32_t)(row_index ? row_index[mr] : mr);
        float v[kStreamMaxKB / 4];
#pragma unroll
        for (int i = 0; i < kStreamMaxKB / 4; ++i) v[i] = a_scales[srow * (uint32_t)KB + min((lane >> 4) + 4 * i, KB - 1)];
#pragma unroll
        for (int i = 0; i < kStreamMaxKB / 4; ++i) sa_lds[((lane >> 4) + 4 * i) * 16 + r] = v[i];
    }
    MTPD_WAIT_VM(0);
    asm volatile("" ::: "memory");
    {
        const uint32_t kl = (uint32_t)min(lane, KB - 1);
        lds_copy4(w_scales + (size_t)(n0 >> 7) * KB, kl * 4u, lds_addr(sw_lds));
    }
#pragma unroll
    for (int j = 0; j < D; ++j) refill(j, min(j, KB - 1));

    // steady state: consume block kb from slot j, refill the slot with block
    // kb + D (clamped)
    int c = 0;
    for (; c + D < KBp; c += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            wait_vm((D - 1) * PER_BLOCK);
            compute(j, c + j);
            refill(j, min(c + D + j, KB - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // last D blocks: nothing more is requested
#pragma unroll
    for (int j = 0; j < D; ++j) {
        wait_vm((D - 1 - j) * PER_BLOCK);
        compute(j, c + j);
        __builtin_amdgcn_sched_barrier(0);
    }
    promote();   // the last block's partials

    // per activation row (4 * (lane / 16) + i) the best key over the wave's
    // NT * 16 vocab rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint64_t best = 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            best = u64_max(best, argmax_key(acc[nt][i], (uint32_t)(n0 + nt * 16 + (lane & 15))));
        best = row16_max_u64(best);
        if ((lane & 15) == 0) red[4 * (lane >> 4) + i] = best;
    }
    __syncthreads();
    uint64_t old = 0;
    if (lane < n_rows) old = merge_key(ws, n_rows, tile, lane, red[lane]);
    const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
    if (lane == 0) last_flag = arrive(ws, tile, total_tiles, dep) ? 1 : 0;
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<64>(ws, n_rows, out_max, out_idx, red);
}

// ---------------------------------------------------------------------------
// 17..64 activation rows: the same weight stream, with the activation shared.
//
// A workgroup is NW waves and stays resident: it takes weight tiles
// t = blockIdx, blockIdx + G, ... (NW*NT*16 vocab rows each), and all its
// tiles' K blocks form one continuous stream, so the rings never drain
// between tiles.  Each wave keeps its own weight ring (as above); the
// activation block (MT*16 rows x 128 bytes) is needed by every wave, so it
// lives in one workgroup ring of the same depth, each wave copying 2*MT/NW of
// its 8-row pieces.  Per block a wave waits for its own copies of that block,
// then a barrier makes every wave's pieces visible; past the barrier all
// waves have finished the previous block, so its slot (activation and
// weight) is refilled with the block D-1 ahead.  The activation scales of all
// rows and the weight-scale rows of all the workgroup's tiles are copied into
// LDS once, before the stream.  At the end of each tile the wave folds its
// per-row best keys into a running maximum in LDS (all tiles share the same
// activation rows); at the end the NW waves' maxima meet, one merge per row,
// arrival, and the last workgroup decodes.
//
// Top-k mode (TOPK): instead of folding per-row maxima, each wave sorts, at
// the end of every tile, the 32 keys of each activation row over its 32
// vocab rows with a bitonic network across the 16 lanes of the row's lane
// group (two keys per lane) and merges them into a running best 32 held in
// registers the same way.  (Spreading those network steps over the next
// tile's blocks measured slower: every block's instruction stream grew.)  After the stream each wave writes the best k
// (<= 32) of every row to its own list in the candidate buffer (no store
// sits inside the stream, whose waits count vector-memory operations), and
// topk_merge_kernel selects each row's best k over all lists.  The keys are the argmax epilogue's, so the
// order is: larger fp32 logit first, lower index first among equal logits.
// ---------------------------------------------------------------------------

constexpr int kRowsMaxTilesPerWg = 16;   // weight-scale rows staged per workgroup
constexpr size_t kLdsPerWorkgroup = 160 * 1024;   // gfx950

// LDS of a rows-kernel shape: the static arrays plus the activation-scale
// table at its largest (H = kStreamMaxH).
constexpr size_t rows_lds_bytes(int mt, int nt, int nw, int d) {
    return (size_t)nw * d * nt * 2 * 64 * 16      // weight rings
           + (size_t)d * mt * 2 * 64 * 16         // activation ring
           + (size_t)kRowsMaxTilesPerWg * kStreamMaxKB * 4
           + (size_t)64 * nw * 8 + 64             // running maxima, flag, alignment
           + (size_t)mt * 16 * kStreamMaxKB * 4;  // activation-scale table
}

// Lane exchange inside groups of 16 lanes for a compile-time xor mask:
// quad permutations (data-parallel moves) for 1 and 2, the LDS swizzle
// network's bit-mask mode for 4 and 8.
template <int M>
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v) {
    int r;
    if constexpr (M == 1)
        r = __builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    else if constexpr (M == 2)
        r = __builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    else
        r = __builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));           // and 0x1F, xor M
    asm volatile("" : "+v"(r));   // pinned where every lane runs it (see dpp_f32)
    return (uint32_t)r;
}
template <int M>
__device__ __forceinline__ uint64_t xor_lanes_u64(uint64_t v) {
    return ((uint64_t)xor_lanes<M>((uint32_t)(v >> 32)) << 32) | xor_lanes<M>((uint32_t)v);
}

// One compare-exchange step of the bitonic network (block size SIZE, partner
// distance M) on N independent 32-key sets held two per lane by the 16 lanes
// of each lane group (lane j holds element j in k0[s], element j + 16 in
// k1[s]); all sets issue their exchanges together so the latencies overlap.
template <int SIZE, int M, int N>
__device__ __forceinline__ void bitonic_step(uint64_t (&k0)[N], uint64_t (&k1)[N], int j) {
    if constexpr (M == 16) {   // elements j and j + 16, one descending block
#pragma unroll
        for (int s = 0; s < N; ++s) {
            const uint64_t hi = u64_max(k0[s], k1[s]), lo = u64_min(k0[s], k1[s]);
            k0[s] = hi;
            k1[s] = lo;
        }
    } else {
        // element e keeps the larger key when it is the lower of its pair
        // inside a descending block (e & SIZE == 0), or the upper inside an
        // ascending one
        const bool lower = (j & M) == 0;
        const bool keep_max0 = lower == ((j & SIZE) == 0);
        const bool keep_max1 = lower == (((j + 16) & SIZE) == 0);
        uint64_t o0[N], o1[N];
#pragma unroll
        for (int s = 0; s < N; ++s) {
            o0[s] = xor_lanes_u64<M>(k0[s]);
            o1[s] = xor_lanes_u64<M>(k1[s]);
        }
#pragma unroll
        for (int s = 0; s < N; ++s) {
            k0[s] = keep_max0 ? u64_max(k0[s], o0[s]) : u64_min(k0[s], o0[s]);
            k1[s] = keep_max1 ? u64_max(k1[s], o1[s]) : u64_min(k1[s], o1[s]);
        }
    }
}

// Reverses the 16 lanes of each lane group (data-parallel row mirror).
__device__ __forceinline__ uint64_t mirror16_u64(uint64_t v) {
    return dpp_u64<0x140>(v);
}

// Merges the descending set (n0, n1) into the descending set (r0, r1),
// keeping the larger 32 keys in descending order: the elementwise maximum of
// r and the reversed n is a bitonic sequence holding the 32 largest keys of
// both, which the last five network steps sort.
template <int N>
__device__ __forceinline__ void merge32_desc(uint64_t (&r0)[N], uint64_t (&r1)[N], const uint64_t (&n0)[N],
                                             const uint64_t (&n1)[N], int j) {
#pragma unroll
    for (int s = 0; s < N; ++s) {
        // element e of the reversed n is n[31 - e]: lane 15 - j, the other half
        r0[s] = u64_max(r0[s], mirror16_u64(n1[s]));
        r1[s] = u64_max(r1[s], mirror16_u64(n0[s]));
    }
    bitonic_step<32, 16, N>(r0, r1, j);
    bitonic_step<32, 8, N>(r0, r1, j);
    bitonic_step<32, 4, N>(r0, r1, j);
    bitonic_step<32, 2, N>(r0, r1, j);
    bitonic_step<32, 1, N>(r0, r1, j);
}

// Sorts N sets of 32 u64 keys (layout as above) into descending order.
template <int N>
__device__ __forceinline__ void sort32_desc(uint64_t (&k0)[N], uint64_t (&k1)[N], int j) {
    bitonic_step<2, 1, N>(k0, k1, j);
    bitonic_step<4, 2, N>(k0, k1, j);
    bitonic_step<4, 1, N>(k0, k1, j);
    bitonic_step<8, 4, N>(k0, k1, j);
    bitonic_step<8, 2, N>(k0, k1, j);
    bitonic_step<8, 1, N>(k0, k1, j);
    bitonic_step<16, 8, N>(k0, k1, j);
    bitonic_step<16, 4, N>(k0, k1, j);
    bitonic_step<16, 2, N>(k0, k1, j);
    bitonic_step<16, 1, N>(k0, k1, j);
    bitonic_step<32, 16, N>(k0, k1, j);
    bitonic_step<32, 8, N>(k0, k1, j);
    bitonic_step<32, 4, N>(k0, k1, j);
    bitonic_step<32, 2, N>(k0, k1, j);
    bitonic_step<32, 1, N>(k0, k1, j);
}

template <int MT, int NT, int NW, int D, bool TOPK>
__global__ __launch_bounds__(64 * NW) void lmhead_stream_rows_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int total_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx,
    ArgmaxWs ws, unsigned long long* __restrict__ cand, int topk)
{
    static_assert(!TOPK || NT == 2, "top-k mode sorts 32 vocab rows per wave");
    constexpr int ROWS = MT * 16;
    constexpr int TROWS = NW * NT * 16;      // vocab rows per tile
    constexpr int WSLOT = NT * 2 * 64;       // uint4s per wave per block
    constexpr int ASLOT = MT * 2 * 64;       // uint4s per activation block
    constexpr int APW = 2 * MT / NW;         // activation pieces each wave copies per block
    static_assert(APW * NW == 2 * MT, "activation pieces must split evenly over the waves");
    constexpr int PER_BLOCK = 2 * NT + APW;
    static_assert((D - 2) * PER_BLOCK <= 63, "vmcnt holds at most 63");
    static_assert(TROWS <= 128 && 128 % TROWS == 0, "a tile sits inside one weight-scale block");
    static_assert(rows_lds_bytes(MT, NT, NW, D) <= kLdsPerWorkgroup, "shape exceeds the LDS of a workgroup");
    __shared__ __align__(16) uint4 wring[NW][D * WSLOT];
    __shared__ __align__(16) uint4 aring[D * ASLOT];
    __shared__ __align__(16) float sw_lds[kRowsMaxTilesPerWg][kStreamMaxKB];
    __shared__ unsigned long long red[64 * NW];   // running per-row maxima, one set per wave
    __shared__ int last_flag;
    extern __shared__ __align__(16) float sa_lds[];   // [KB][ROWS], block-major

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int KB = H >> 7;
    const int G = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    const int ntiles = (total_tiles - b + G - 1) / G;   // this workgroup's tiles: b, b+G, ...
    const int nunits = ntiles * KB;

    uint32_t woff[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int r = 8 * q + (lane >> 3);
            woff[nt][q] = (uint32_t)(wave * NT * 16 + nt * 16 + r) * (uint32_t)H +
                          (uint32_t)ring_pos(r, lane & 7) * 16u;
        }
    // activation copies: piece p = wave + NW*i covers rows 8p..8p+7 (row tile
    // p/2, half p%2), clamped to the last row
    uint32_t aoff[APW];
#pragma unroll
    for (int i = 0; i < APW; ++i) {
        const int p = wave + NW * i;
        const int r16 = 8 * (p & 1) + (lane >> 3);
        const int m = min(8 * p + (lane >> 3), n_rows - 1);
        aoff[i] = (uint32_t)(row_index ? row_index[m] : m) * (uint32_t)H + (uint32_t)ring_pos(r16, lane & 7) * 16u;
    }
    // the activation-scale table, block-major [KB][ROWS] so a lane's four
    // fragment rows of a block are one 16-byte read and the four lane groups
    // hit distinct banks: thread t fills row t % ROWS.  Register loads, all
    // completed (and the table published) before any copy is issued.
    {
        constexpr int THREADS = 64 * NW;
        static_assert(THREADS % ROWS == 0, "each thread fills one row of the table");
        const int row = t % ROWS;
        const int m = min(row, n_rows - 1);
        const uint32_t srow = (uint32_t)(row_index ? row_index[m] : m);
        for (int kb = t / ROWS; kb < KB; kb += THREADS / ROWS) sa_lds[kb * ROWS + row] = a_scales[srow * (uint32_t)KB + kb];
    }
    __syncthreads();

    const int fr = lane & 15, fg = lane >> 4;
    const int fpos0 = fr * 8 + ring_pos(fr, fg);
    const int fpos1 = fr * 8 + ring_pos(fr, fg + 4);
    const uint32_t wring0 = lds_addr(&wring[wave][0]);
    const uint32_t aring0 = lds_addr(aring);

    // unit u = (tile index i, block kb); refills walk the units with their
    // own counters (clamped to the last unit)
    auto refill = [&](int j, int i, int kb) {
        const int tile = b + i * G;
        const uint8_t* wb = w_codes + (size_t)tile * TROWS * (size_t)H + (size_t)kb * kBlock;
        const uint8_t* ab = a_codes + (size_t)kb * kBlock;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 2; ++q) lds_copy16_stream(wb, woff[nt][q], wring0 + (uint32_t)(j * WSLOT + (nt * 2 + q) * 64) * 16u);
#pragma unroll
        for (int i2 = 0; i2 < APW; ++i2)
            lds_copy16(ab, aoff[i2], aring0 + (uint32_t)(j * ASLOT + (wave + NW * i2) * 64) * 16u);
    };

    // prologue: the weight-scale rows of the workgroup's tiles (lanes past
    // KB idle), then units 0..D-2
    if (lane < KB) {
        for (int i = wave; i < ntiles; i += NW)
            lds_copy4(w_scales + (size_t)((b + i * G) * TROWS >> 7) * KB, (uint32_t)lane * 4u, lds_addr(&sw_lds[i][0]));
    }
    if (lane < ROWS) red[wave * 64 + lane] = 0;
    int ri = 0, rkb = 0;   // next unit to request
    auto next_req = [&]() {
        const int i = ri, kb = rkb;
        if (ri * KB + rkb < nunits - 1) {
            if (++rkb == KB) { rkb = 0; ++ri; }
        }
        return make_int2(i, kb);
    };
#pragma unroll
    for (int j = 0; j < D - 1; ++j) {
        const int2 u = next_req();
        refill(j, u.x, u.y);
    }

    float acc[MT][NT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.f;

    // top-k mode: the running best 32 keys per activation row (layout of
    // sort32_desc; key 0 is below every real key)
    constexpr int NS = TOPK ? MT * 4 : 1;
    uint64_t run0[NS], run1[NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
        run0[s2] = 0;
        run1[s2] = 0;
    }

    // each unit's partials are promoted one unit late (pp, pf): the FMAs of
    // unit u run beside the MFMAs of unit u + 1 instead of waiting for fresh
    // results; the order of every sum is unchanged
    v4f pp[MT][NT];
    float4 pf[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        pf[mt] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pp[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    auto promote = [&](int mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            acc[mt][nt][0] = fmaf(pp[mt][nt][0], pf[mt].x, acc[mt][nt][0]);
            acc[mt][nt][1] = fmaf(pp[mt][nt][1], pf[mt].y, acc[mt][nt][1]);
            acc[mt][nt][2] = fmaf(pp[mt][nt][2], pf[mt].z, acc[mt][nt][2]);
            acc[mt][nt][3] = fmaf(pp[mt][nt][3], pf[mt].w, acc[mt][nt][3]);
        }
    };
    auto flush = [&]() {   // promote the pending unit and clear it
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            promote(mt);
            pf[mt] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto compute = [&](int j, int i, int kb, bool live) {
        const float swl = sw_lds[i][kb];
        const float sw = live ? swl : 0.f;
        const uint4* tw = &wring[wave][j * WSLOT];
        v8i bf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bf[nt] = make_frag(tw[nt * 128 + fpos0], tw[nt * 128 + fpos1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4* ta = &aring[j * ASLOT + mt * 128];
            const v8i af = make_frag(ta[fpos0], ta[fpos1]);
            const float4 sa4 = *reinterpret_cast<const float4*>(&sa_lds[kb * ROWS + mt * 16 + 4 * fg]);
            v4f p[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) p[nt] = mfma_e4m3(af, bf[nt]);
            promote(mt);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) pp[mt][nt] = p[nt];
            pf[mt] = make_float4(sa4.x * sw, sa4.y * sw, sa4.z * sw, sa4.w * sw);
        }
    };
    // a finished tile: per-row best over this wave's columns, folded into the
    // wave's running maxima (top-k mode: the wave's best k per row, written
    // to its list); the accumulators restart
    auto fold = [&](int i) {
        flush();   // the tile's last unit
        const int n0 = (b + i * G) * TROWS + wave * NT * 16;
        if constexpr (TOPK) {
            const int j = lane & 15;
            uint64_t k0[NS], k1[NS];   // set mt * 4 + r: activation rows mt * 16 + 4 * (lane / 16) + r
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    k0[mt * 4 + r] = argmax_key(acc[mt][0][r], (uint32_t)(n0 + j));
                    k1[mt * 4 + r] = argmax_key(acc[mt][1][r], (uint32_t)(n0 + 16 + j));
                    acc[mt][0][r] = 0.f;
                    acc[mt][1][r] = 0.f;
                }
            sort32_desc<NS>(k0, k1, j);
            merge32_desc<NS>(run0, run1, k0, k1, j);
            return;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint64_t best = 0;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    best = u64_max(best, argmax_key(acc[mt][nt][r], (uint32_t)(n0 + nt * 16 + (lane & 15))));
                    acc[mt][nt][r] = 0.f;
                }
                best = row16_max_u64(best);
                if ((lane & 15) == 0) {
                    unsigned long long* slot = &red[wave * 64 + mt * 16 + 4 * (lane >> 4) + r];
                    *slot = u64_max(*slot, best);
                }
            }
    };

    // units in rounds of D so ring slots are compile-time; the last round is
    // padded with repeats of the last unit (zero weight-scale factor)
    int ci = 0, ckb = 0;   // unit being consumed
    const int nup = (nunits + D - 1) / D * D;
    for (int c = 0; c < nup; c += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            wait_vm((D - 2) * PER_BLOCK);   // this wave's copies of this unit
            __builtin_amdgcn_s_barrier();   // everyone's; and everyone is past the previous unit
            asm volatile("" ::: "memory");
            {
                const int2 u = next_req();
                refill((j + D - 1) % D, u.x, u.y);
            }
            const bool live = c + j < nunits;
            compute(j, ci, ckb, live);
            if (live && ckb == KB - 1) fold(ci);
            if (live && ++ckb == KB) { ckb = 0; ++ci; }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    MTPD_WAIT_VM(0);   // the clamped tail refills, before LDS is reused
    __syncthreads();
    if constexpr (TOPK) {   // this wave's list: the best k of every row
        const int j = lane & 15;
        const size_t list = (size_t)b * NW + wave;
        const size_t n_lists = (size_t)G * NW;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mt * 16 + 4 * (lane >> 4) + r;
                if (row < n_rows) {
                    unsigned long long* dst = cand + ((size_t)row * n_lists + list) * (size_t)topk;
                    if (j < topk) dst[j] = run0[mt * 4 + r];
                    if (j + 16 < topk) dst[j + 16] = run1[mt * 4 + r];
                }
            }
        return;   // the lists are merged by topk_merge_kernel
    }

    if (wave == 0) {
        uint64_t old = 0;
        if (lane < ROWS && lane < n_rows) {
            uint64_t k = red[lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) k = u64_max(k, red[w * 64 + lane]);
            old = merge_key(ws, n_rows, b, lane, k);
        }
        const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
        if (lane == 0) last_flag = arrive(ws, b, G, dep) ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<64 * NW>(ws, n_rows, out_max, out_idx, red);
}

#define MTPD_ROWS_CONFIGS(X) X(4, 2, 4, 4) X(4, 2, 4, 5) X(4, 1, 8, 4) X(4, 2, 4, 3) X(4, 1, 4, 4) X(4, 1, 4, 3) X(2, 2, 4, 4) X(2, 2, 4, 6) X(2, 1, 4, 6) X(2, 1, 4, 4) X(4, 1, 4, 6)

bool rows_config_compiled(int mt, int nt, int nw, int d) {
#define MTPD_X(a, b, c2, e) if (mt == a && nt == b && nw == c2 && d == e) return true;
    MTPD_ROWS_CONFIGS(MTPD_X)
#undef MTPD_X
    return false;
}

hipError_t launch_lmhead_rows(const LmheadArgs& a, int mt, int nt, int nw, int d, int cus, hipStream_t stream) {
    const int64_t tiles = a.V / (16 * nt * nw);
    if (tiles > 0x7FFFFFFF || a.H > kStreamMaxH || a.n_rows > 16 * mt) return hipErrorInvalidValue;
    // one resident workgroup per CU, at most kRowsMaxTilesPerWg tiles each
    int64_t grid = std::min<int64_t>(tiles, cus);
    grid = std::max<int64_t>(grid, (tiles + kRowsMaxTilesPerWg - 1) / kRowsMaxTilesPerWg);
    const size_t lds = (size_t)(16 * mt) * (size_t)(a.H / kBlock) * sizeof(float);
    // never dispatch a shape whose LDS (static + the scale table) does not fit
    // a workgroup: the dispatch would be rejected by the device
    auto fits = [&](const void* kernel) {
        hipFuncAttributes attr;
        if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return false;
        int dev = 0, cap = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cap, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return false;
        return attr.sharedSizeBytes + lds <= (size_t)cap;
    };
#define MTPD_X(p, q, r, u)                                                                                    \
    if (mt == p && nt == q && nw == r && d == u) {                                                           \
        if (!fits(reinterpret_cast<const void*>(&lmhead_stream_rows_kernel<p, q, r, u, false>)))            \
            return hipErrorInvalidConfiguration;                                                             \
        hipLaunchKernelGGL((lmhead_stream_rows_kernel<p, q, r, u, false>), dim3((unsigned)grid), dim3(64 * r), \
                           lds, stream, a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes,         \
                           a.w_scales, (int)a.H, (int)tiles, a.out_max, a.out_idx,                            \
                           argmax_ws(a.workspace, a.n_rows), nullptr, 0);                                     \
        return hipGetLastError();                                                                            \
    }
    MTPD_ROWS_CONFIGS(MTPD_X)
#undef MTPD_X
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// 17-64 rows with K outermost.  The tile-by-tile kernel above copies the
// whole activation (64 rows x H bytes) into LDS once per 128-row weight tile,
// a third of its copy traffic at c = 64.  Here a workgroup walks K blocks in
// the outer loop and its TMAX tiles (b, b + G, ...) in the inner one, keeping
// TMAX tiles' accumulators in registers, so each activation block is copied
// once per workgroup and shared by all its tiles, and the waves meet at one
// barrier per K block instead of one per unit.
//
//  - Units (block kb, tile slot i), i fastest; slots at or past the
//    workgroup's tile count are dead (their copies repeat its last tile's
//    block, their factor is zero), so every block walks exactly TMAX units
//    and every register index is a compile-time constant.
//  - Each unit's copies: the wave's NT weight tiles (2 * NT copies) and one
//    more, either a 1 KB piece of activation block kb + 1 (the first
//    2 * MT / NW units of the block carry its pieces) or a 4-byte placeholder,
//    so every unit issues the same number of vector-memory operations and
//    the waits stay compile-time counts.  Activation blocks rotate through
//    three slots: the block in use, the next one, and the one being filled
//    (requests run at most TMAX units ahead, so block kb + 1 is requested no
//    earlier than block kb - 1 is in use, after the barrier that ends block
//    kb - 2).
//  - Each unit's partials are promoted at once; the keys of all tiles are
//    formed after the stream, per lane over the tiles first and then one
//    16-lane maximum per row.
// ---------------------------------------------------------------------------

template <int MT, int NT, int NW, int D, int TMAX>
__global__ __launch_bounds__(64 * NW) void lmhead_kouter_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int total_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx, ArgmaxWs ws)
{
    constexpr int ROWS = MT * 16;
    constexpr int TROWS = NW * NT * 16;      // vocab rows per tile
    constexpr int WSLOT = NT * 2 * 64;       // uint4s per wave per unit
    constexpr int ASLOT = MT * 2 * 64;       // uint4s per activation block
    constexpr int DA = 3;                    // activation block slots
    constexpr int PIECES = 2 * MT;           // 1 KB copies per activation block
    constexpr int PW = PIECES / NW;          // pieces per wave: carried by units 0 .. PW - 1 of a block
    static_assert(PW * NW == PIECES && PW <= TMAX, "activation pieces must split evenly over the waves");
    static_assert(D >= 2 && D - 1 <= TMAX, "requests run at most TMAX units ahead");
    constexpr int PER_UNIT = 2 * NT + 1;
    static_assert((D - 2) * PER_UNIT <= 63, "vmcnt holds at most 63");
    static_assert(TROWS <= 128 && 128 % TROWS == 0, "a tile sits inside one weight-scale block");
    __shared__ __align__(16) uint4 wring[NW][D * WSLOT];
    __shared__ __align__(16) uint4 aring[DA * ASLOT];
    __shared__ __align__(16) float sw_lds[TMAX][kStreamMaxKB];
    __shared__ unsigned int sink[NW][64];    // placeholder copies land here, never read
    __shared__ unsigned long long red[64 * NW];
    __shared__ int last_flag;
    extern __shared__ __align__(16) float sa_lds[];   // [KB][ROWS], block-major

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int KB = H >> 7;
    const int G = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    const int ntiles = (total_tiles - b + G - 1) / G;   // 1 .. TMAX (the host sizes the grid)

    uint32_t woff[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int r = 8 * q + (lane >> 3);
            woff[nt][q] = (uint32_t)(wave * NT * 16 + nt * 16 + r) * (uint32_t)H +
                          (uint32_t)ring_pos(r, lane & 7) * 16u;
        }
    // this wave's activation pieces p = wave + NW * j (rows 8p .. 8p + 7 of
    // row tile p / 2, half p % 2), clamped to the last row
    uint32_t aoff[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int p = wave + NW * j;
        const int r16 = 8 * (p & 1) + (lane >> 3);
        const int m = min(8 * p + (lane >> 3), n_rows - 1);
        aoff[j] = (uint32_t)(row_index ? row_index[m] : m) * (uint32_t)H + (uint32_t)ring_pos(r16, lane & 7) * 16u;
    }
    {
        constexpr int THREADS = 64 * NW;
        static_assert(THREADS % ROWS == 0, "each thread fills one row of the table");
        const int row = t % ROWS;
        const int m = min(row, n_rows - 1);
        const uint32_t srow = (uint32_t)(row_index ? row_index[m] : m);
        for (int kb = t / ROWS; kb < KB; kb += THREADS / ROWS) sa_lds[kb * ROWS + row] = a_scales[srow * (uint32_t)KB + kb];
    }
    __syncthreads();

    const int fr = lane & 15, fg = lane >> 4;
    const int fpos0 = fr * 8 + ring_pos(fr, fg);
    const int fpos1 = fr * 8 + ring_pos(fr, fg + 4);
    const uint32_t wring0 = lds_addr(&wring[wave][0]);
    const uint32_t aring0 = lds_addr(aring);
    const uint32_t sink0 = lds_addr(&sink[wave][0]);

    // requests walk the units with their own counters, clamped at the last
    // unit (units past it repeat it into slots that are never read)
    int rkb = 0, ri = 0;
    auto refill = [&](int slot) {
        const int kb = rkb, i = ri;
        const int tile = b + min(i, ntiles - 1) * G;
        const uint8_t* wb = w_codes + (size_t)tile * TROWS * (size_t)H + (size_t)kb * kBlock;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                lds_copy16_stream(wb, woff[nt][q], wring0 + (uint32_t)(slot * WSLOT + (nt * 2 + q) * 64) * 16u);
        if (i < PW && kb + 1 < KB) {
            const uint32_t dst = aring0 + (uint32_t)(((kb + 1) % DA) * ASLOT + (wave + NW * i) * 64) * 16u;
            uint32_t ao = aoff[0];
#pragma unroll
            for (int j = 1; j < PW; ++j) ao = i == j ? aoff[j] : ao;
            lds_copy16(a_codes + (size_t)(kb + 1) * kBlock, ao, dst);
        } else {
            lds_copy4(a_scales, 0u, sink0);
        }
        if (kb < KB - 1 || i < TMAX - 1) {
            if (++ri == TMAX) { ri = 0; ++rkb; }
        }
    };

    // prologue: the tiles' weight-scale rows (lanes past KB idle), activation
    // block 0, then units 0 .. D - 2
    if (lane < KB) {
        for (int i = wave; i < ntiles; i += NW)
            lds_copy4(w_scales + (size_t)((b + i * G) * TROWS >> 7) * KB, (uint32_t)lane * 4u, lds_addr(&sw_lds[i][0]));
    }
#pragma unroll
    for (int j = 0; j < PW; ++j) lds_copy16(a_codes, aoff[j], aring0 + (uint32_t)((wave + NW * j) * 64) * 16u);
    if (lane < ROWS) red[wave * 64 + lane] = 0;
#pragma unroll
    for (int j = 0; j < D - 1; ++j) refill(j);

    float acc[TMAX][MT][NT][4];
#pragma unroll
    for (int i = 0; i < TMAX; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][mt][nt][r] = 0.f;
    v4f pp[MT][NT];
    float4 pf[MT];
    // a unit's partials into tile slot ip's accumulators (at once: carrying
    // them to the next unit, as the kernel above does, costs registers this
    // kernel does not have)
    auto promote = [&](int ip, int mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            acc[ip][mt][nt][0] = fmaf(pp[mt][nt][0], pf[mt].x, acc[ip][mt][nt][0]);
            acc[ip][mt][nt][1] = fmaf(pp[mt][nt][1], pf[mt].y, acc[ip][mt][nt][1]);
            acc[ip][mt][nt][2] = fmaf(pp[mt][nt][2], pf[mt].z, acc[ip][mt][nt][2]);
            acc[ip][mt][nt][3] = fmaf(pp[mt][nt][3], pf[mt].w, acc[ip][mt][nt][3]);
        }
    };

    int cslot = 0;
    v8i af[MT];       // the block's activation fragments, read at its first unit
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
            wait_vm((D - 2) * PER_UNIT);   // this wave's copies of this unit (and all older ones)
            if (i == 0) {                  // everyone's copies of activation block kb; all past block kb - 1
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            refill(cslot == 0 ? D - 1 : cslot - 1);
            if (i == 0) {
                const uint4* ta = &aring[(kb % DA) * ASLOT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) af[mt] = make_frag(ta[mt * 128 + fpos0], ta[mt * 128 + fpos1]);
            }
            const float sw = i < ntiles ? sw_lds[i][kb] : 0.f;
            const uint4* tw = &wring[wave][cslot * WSLOT];
            v8i bf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bf[nt] = make_frag(tw[nt * 128 + fpos0], tw[nt * 128 + fpos1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 sa4 = *reinterpret_cast<const float4*>(&sa_lds[kb * ROWS + mt * 16 + 4 * fg]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) pp[mt][nt] = mfma_e4m3(af[mt], bf[nt]);
                pf[mt] = make_float4(sa4.x * sw, sa4.y * sw, sa4.z * sw, sa4.w * sw);
                promote(i, mt);
            }
            cslot = cslot + 1 == D ? 0 : cslot + 1;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    MTPD_WAIT_VM(0);   // the clamped tail requests, before LDS is reused

    // per-row best over this wave's columns of every live tile: per lane
    // over the tiles first, then one 16-lane maximum per row
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint64_t best = 0;
#pragma unroll
            for (int i = 0; i < TMAX; ++i) {
                const uint32_t n0 = (uint32_t)((b + i * G) * TROWS + wave * NT * 16 + (lane & 15));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const uint64_t k = argmax_key(acc[i][mt][nt][r], n0 + (uint32_t)(nt * 16));
                    best = i < ntiles ? u64_max(best, k) : best;
                }
            }
            best = row16_max_u64(best);
            if ((lane & 15) == 0) red[wave * 64 + mt * 16 + 4 * (lane >> 4) + r] = best;
            __builtin_amdgcn_sched_barrier(0);
        }
    __syncthreads();
    if (wave == 0) {
        uint64_t old = 0;
        if (lane < ROWS && lane < n_rows) {
            uint64_t k = red[lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) k = u64_max(k, red[w * 64 + lane]);
            old = merge_key(ws, n_rows, b, lane, k);
        }
        const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
        if (lane == 0) last_flag = arrive(ws, b, G, dep) ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<64 * NW>(ws, n_rows, out_max, out_idx, red);
}

#define MTPD_KOUTER_CONFIGS(X) X(4, 1, 8, 4, 4) X(4, 2, 4, 5, 5)

bool kouter_choose(int mt, int64_t V, int cus, KouterTile* out) {
    // the plan override may rule the kernel out or pin one shape (testing)
    const PlanOverride& po = plan_override();
    KouterTile want{0, 0, 0, 0};
    if (po.kouter < 0) return false;
    if (po.kouter > 0) want = KouterTile{po.kouter_shape[0], po.kouter_shape[1], po.kouter_shape[2], po.kouter_shape[3]};
#define MTPD_X(a, b2, c2, e2, f)                                                                              \
    if (mt == a && V % (16 * b2 * c2) == 0 && (want.nt == 0 || (want.nt == b2 && want.nw == c2 &&            \
                                                                  want.d == e2 && want.tmax == f))) {        \
        const int64_t tiles = V / (16 * b2 * c2), g = std::min<int64_t>(tiles, cus);                         \
        if (tiles >= 2 * g - 1 && (tiles + g - 1) / g == f) {                                                 \
            *out = KouterTile{b2, c2, e2, f};                                                                 \
            return true;                                                                                      \
        }                                                                                                     \
    }
    MTPD_KOUTER_CONFIGS(MTPD_X)
#undef MTPD_X
    return false;
}

hipError_t launch_lmhead_kouter(const LmheadArgs& a, int mt, int nt, int nw, int d, int tmax, int cus,
                                hipStream_t stream) {
    const int64_t tiles = a.V / (16 * nt * nw);
    if (tiles < 1 || tiles > 0x7FFFFFFF || a.H > kStreamMaxH || a.n_rows > 16 * mt) return hipErrorInvalidValue;
    const int64_t grid = std::min<int64_t>(tiles, cus);
    if ((tiles + grid - 1) / grid > tmax) return hipErrorInvalidValue;   // at most tmax tiles per workgroup
    const size_t lds = (size_t)(16 * mt) * (size_t)(a.H / kBlock) * sizeof(float);
#define MTPD_X(p, q, r, u, v)                                                                                \
    if (mt == p && nt == q && nw == r && d == u && tmax == v) {                                              \
        hipLaunchKernelGGL((lmhead_kouter_kernel<p, q, r, u, v>), dim3((unsigned)grid), dim3(64 * r), lds,   \
                           stream, a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales, \
                           (int)a.H, (int)tiles, a.out_max, a.out_idx, argmax_ws(a.workspace, a.n_rows));   \
        return hipGetLastError();                                                                            \
    }
    MTPD_KOUTER_CONFIGS(MTPD_X)
#undef MTPD_X
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Top-k (k <= 32): the rows kernel in top-k mode writes, per activation row,
// one sorted list of the best k keys for every wave of its (persistent)
// grid.  One
// workgroup per row then bounds the row's k-th key from below by the k-th
// largest of its threads' best list heads, gathers every key at or above
// that bound into LDS (lists are sorted, so each is read only down to its
// first smaller key) and places each gathered key by counting the larger
// ones.  If nearly equal logits put more than 2048 keys above the bound, a
// slower selection (private best-32 per thread, then k rounds of a
// workgroup maximum) takes over.
// ---------------------------------------------------------------------------

constexpr int kTopkMax = 32;
constexpr int kTopkRows = 64;      // activation rows per rows-kernel pass
constexpr int kTopkListRows = 128; // vocab rows per tile (NT = 2, NW = 4)

__global__ __launch_bounds__(256) void topk_merge_kernel(const unsigned long long* __restrict__ cand, int n_lists,
                                                         int k, float* __restrict__ out_val,
                                                         int32_t* __restrict__ out_idx)
{
    constexpr int kCap = 2048;   // candidates kept in LDS for the rank selection
    __shared__ unsigned long long buf[kCap];
    __shared__ unsigned long long heads[256];
    __shared__ unsigned long long wred[4];
    __shared__ unsigned long long thr;
    __shared__ int count;
    const int row = (int)blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const unsigned long long* base = cand + (size_t)row * (size_t)n_lists * (size_t)k;
    float* vrow = out_val + (size_t)row * k;
    int32_t* irow = out_idx + (size_t)row * k;

    // 1. a lower bound T of the row's k-th key: each thread's best list head
    //    (lists are sorted), and the k-th largest of those 256 maxima (k
    //    distinct keys are at least that large).  Keys are unique and
    //    nonzero; a thread without lists offers 0.
    uint64_t h = 0;
    for (int l = t; l < n_lists; l += 256) h = u64_max(h, base[(size_t)l * k]);
    heads[t] = h;
    if (t == 0) {
        thr = 0;
        count = 0;
    }
    __syncthreads();
    if (h != 0) {
        int rank = 0;
        for (int q = 0; q < 256; ++q) rank += heads[q] > h ? 1 : 0;
        if (rank == k - 1) thr = h;
    }
    __syncthreads();
    const uint64_t T = thr;

    // 2. every key >= T into LDS (a list is left at its first smaller key)
    for (int l = t; l < n_lists; l += 256) {
        const unsigned long long* lst = base + (size_t)l * k;
        for (int e = 0; e < k; ++e) {
            const uint64_t x = lst[e];
            if (x < T) break;
            const int pos = atomicAdd(&count, 1);
            if (pos < kCap) buf[pos] = x;
        }
    }
    __syncthreads();
    const int n = count;

    if (n <= kCap) {
        // 3. rank selection: a key's position is the number of larger keys
        for (int c = t; c < n; c += 256) {
            const uint64_t x = buf[c];
            int rank = 0;
            for (int q = 0; q < n; ++q) rank += buf[q] > x ? 1 : 0;
            if (rank < k) {
                vrow[rank] = key_value(x);
                irow[rank] = key_index(x);
            }
        }
        return;
    }

    // 3'. too many keys >= T (nearly equal logits): a private best-32 per
    //     thread over them, then the k best of the 256 private heads
    uint64_t best[kTopkMax];
#pragma unroll
    for (int p = 0; p < kTopkMax; ++p) best[p] = 0;
    for (int l = t; l < n_lists; l += 256) {
        const unsigned long long* lst = base + (size_t)l * k;
        for (int e = 0; e < k; ++e) {
            uint64_t x = lst[e];
            if (x < T || x <= best[kTopkMax - 1]) break;   // sorted list: nothing after it enters either
#pragma unroll
            for (int p = 0; p < kTopkMax; ++p) {
                const uint64_t hi = u64_max(best[p], x);
                x = u64_min(best[p], x);
                best[p] = hi;
            }
        }
    }
    for (int e = 0; e < k; ++e) {
        uint64_t m = best[0];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = u64_max(m, shfl_xor_u64(m, off));
        if (lane == 0) wred[wave] = m;
        __syncthreads();
        const uint64_t bm = u64_max(u64_max(wred[0], wred[1]), u64_max(wred[2], wred[3]));
        __syncthreads();   // every thread has read wred before the next round rewrites it
        if (best[0] == bm) {   // keys are unique: exactly one thread holds the winner
#pragma unroll
            for (int p = 0; p < kTopkMax - 1; ++p) best[p] = best[p + 1];
            best[kTopkMax - 1] = 0;
        }
        if (t == 0) {
            vrow[e] = key_value(bm);
            irow[e] = key_index(bm);
        }
    }
}

bool topk_supported(int64_t H, int64_t a_rows) { return H <= kStreamMaxH && a_rows * H <= ((int64_t)1 << 32); }

size_t topk_workspace_bytes(int64_t n_rows, int64_t V, int64_t k) {
    if (n_rows <= 0) return 0;
    const int64_t rows = std::min<int64_t>(n_rows, kTopkRows);
    const int64_t lists = V / kTopkListRows * 4;
    return ((size_t)rows * (size_t)lists * (size_t)k * 8 + 255) & ~(size_t)255;
}

hipError_t launch_lmhead_topk(const LmheadArgs& a, int k, float* out_val, int32_t* out_idx, int cus,
                              hipStream_t stream) {
    const int64_t tiles = a.V / kTopkListRows;
    if (a.n_rows < 1 || a.n_rows > kTopkRows || k < 1 || k > kTopkMax || tiles > 0x7FFFFFFF ||
        !topk_supported(a.H, a.a_rows))
        return hipErrorInvalidValue;
    int64_t grid = std::min<int64_t>(tiles, cus);
    grid = std::max<int64_t>(grid, (tiles + kRowsMaxTilesPerWg - 1) / kRowsMaxTilesPerWg);
    const int mt = a.n_rows <= 32 ? 2 : 4;
    const size_t lds = (size_t)(16 * mt) * (size_t)(a.H / kBlock) * sizeof(float);
    unsigned long long* cand = reinterpret_cast<unsigned long long*>(a.workspace);
    auto fits = [&](const void* kernel) {
        hipFuncAttributes attr;
        if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return false;
        int dev = 0, cap = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cap, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return false;
        return attr.sharedSizeBytes + lds <= (size_t)cap;
    };
#define MTPD_TOPK_LAUNCH(M)                                                                                   \
    {                                                                                                          \
        if (!fits(reinterpret_cast<const void*>(&lmhead_stream_rows_kernel<M, 2, 4, 3, true>)))              \
            return hipErrorInvalidConfiguration;                                                               \
        hipLaunchKernelGGL((lmhead_stream_rows_kernel<M, 2, 4, 3, true>), dim3((unsigned)grid), dim3(256), lds, \
                           stream, a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales,    \
                           (int)a.H, (int)tiles, nullptr, nullptr, ArgmaxWs{}, cand, k);                       \
    }
    if (mt == 2)
        MTPD_TOPK_LAUNCH(2)
    else
        MTPD_TOPK_LAUNCH(4)
#undef MTPD_TOPK_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)a.n_rows), dim3(256), 0, stream, cand, (int)(grid * 4), k,
                       out_val, out_idx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The whole draft tail for one row (decode at concurrency 1) in one kernel.
//
// One resident workgroup of four waves per CU takes the 16-row weight tiles
// t = blockIdx, blockIdx + G, ...; each wave streams a quarter of every
// tile's K blocks through its own ring, and all of the workgroup's tiles form
// one continuous stream per wave, so the rings never drain between tiles.
// At the end of each tile the four partial sums meet in LDS and are added in
// wave order into a running per-lane best key.
//
// Before the stream the workgroup computes the row's residual add + RMSNorm
// + E4M3 packing itself (norm_quant_kernel's body for one row, thread for
// thread: same per-thread fma order, same wave sum, same fixed-order sum of
// the four wave totals), so the packed row and the bf16 hidden are
// bit-identical to the two-kernel path; the packed row stays in LDS as the
// MFMA activation (every fragment row reads row 0).  The norm inputs (bf16
// hidden and residual, fp32 norm weight) reach LDS by direct copies issued
// before the weight ring, so the norm waits only for them while the ring
// fills (the vector-memory counter is in order).  Workgroup 0 writes the
// row's outputs after its stream.
//
// The same kernel is the LM head alone for one packed row (hidden == NULL):
// the row's codes and scales reach LDS by direct copies in place of the norm
// inputs, and nothing but the (max, index) pair is written.
// ---------------------------------------------------------------------------

constexpr int kTail1MaxH = 8192;   // NSTEP <= 4 steps of 2048 columns
constexpr int kTail1D = 6;         // ring depth per wave
constexpr int kTail1MaxTiles = 16; // tiles per workgroup (one staged weight-scale row each)

// NSTEP 2048-column steps of the norm (3 up to H = 6144, 4 up to 8192): the
// step count of norm_quant_kernel for that H or more, whose extra steps hold
// s = 0 and add exact zeros to the sum of squares, so the norm stays
// bit-identical to the two-launch path
template <int NSTEP>
__global__ __launch_bounds__(256) void draft_tail1_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ residual,
    const float* __restrict__ gamma, float eps, int H,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int total_tiles,
    uint16_t* __restrict__ out_hidden, uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx, ArgmaxWs ws,
    const uint8_t* __restrict__ act_codes, const float* __restrict__ act_scales,
    const int32_t* __restrict__ row_index)
{
    constexpr int D = kTail1D;
    constexpr int SLOT = 2 * 64;             // one 16-row weight tile (uint4s)
    constexpr int PER_BLOCK = 2;
    static_assert(NSTEP * 2048 <= kTail1MaxH, "the norm's steps cover at most kTail1MaxH columns");
    static_assert((D - 1) * PER_BLOCK <= 63, "vmcnt holds at most 63");
    __shared__ __align__(16) uint4 ring[4][D * SLOT];
    // norm inputs as copied: per step k, hidden and residual in column order;
    // the norm weight as two 1 KB halves per (step, wave): lane l's columns
    // 8t..8t+3 in the first, 8t+4..8t+7 in the second
    __shared__ __align__(16) uint4 h_lds[NSTEP * 256];
    __shared__ __align__(16) uint4 r_lds[NSTEP * 256];
    __shared__ __align__(16) uint4 g_lds[NSTEP * 2 * 256];
    __shared__ __align__(16) uint8_t a_lds[NSTEP * 2048];
    __shared__ __align__(16) float sa_lds[kStreamMaxKB];
    __shared__ __align__(16) float sw_lds[kTail1MaxTiles][kStreamMaxKB];
    __shared__ float part[2][4][16];
    __shared__ float wave_sum[4];
    __shared__ unsigned long long red[256];
    __shared__ int last_flag;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int KB = H >> 7;
    const int G = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    const bool fused = hidden != nullptr;   // else the LM head alone on a packed row
    const int ntiles = (total_tiles - b + G - 1) / G;   // this workgroup's tiles: b, b + G, ...
    // this wave's K blocks of every tile [kb0, kb1); every wave walks NBU
    // units per tile (units past its range are dead: zero factor).  With
    // fewer than four K blocks some waves own none (nb = 0): their units read
    // block kb0 (< KB, real data, so the dead partial is a finite zero)
    const int kb0 = (wave * KB) >> 2, kb1 = ((wave + 1) * KB) >> 2;
    const int nb = kb1 - kb0;
    const int NBU = (KB + 3) >> 2;
    const int nunits = ntiles * NBU;
    const int nup = (nunits + D - 1) / D * D;

    uint32_t woff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 8 * q + (lane >> 3);
        woff[q] = (uint32_t)r * (uint32_t)H + (uint32_t)ring_pos(r, lane & 7) * 16u;
    }
    const int fr = lane & 15, fg = lane >> 4;
    const int fpos0 = fr * 8 + ring_pos(fr, fg);
    const int fpos1 = fr * 8 + ring_pos(fr, fg + 4);
    const uint32_t ring0 = lds_addr(&ring[wave][0]);
    // unit u: tile i = u / NBU, block slot j = u % NBU of this wave's range
    // (clamped: units past the last request the last one again)
    auto refill = [&](int slot, int u) {
        const int uc = min(u, nunits - 1);
        const int i = uc / NBU, j = uc - i * NBU;
        const int kb = kb0 + max(min(j, nb - 1), 0);
        const uint8_t* wb = w_codes + (size_t)(b + i * G) * 16 * (size_t)H + (size_t)kb * kBlock;
#pragma unroll
        for (int q = 0; q < 2; ++q) lds_copy16_stream(wb, woff[q], ring0 + (uint32_t)(slot * SLOT + q * 64) * 16u);
    };

    // 1. copies, oldest first: the norm inputs (thread t's 16-byte pieces of
    //    columns k*2048 + 8t, clamped into the row), the weight-scale rows of
    //    the workgroup's tiles (first and last tile's row span, lanes past KB
    //    idle), then the first D-1 units of the ring
    if (fused) {
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
            const uint32_t cc = (uint32_t)min(k * 2048 + t * 8, H - 8);
            const uint32_t dst = (uint32_t)(k * 256 + wave * 64) * 16u;
            lds_copy16(reinterpret_cast<const uint8_t*>(hidden), cc * 2u, lds_addr(h_lds) + dst);
            lds_copy16(reinterpret_cast<const uint8_t*>(residual), cc * 2u, lds_addr(r_lds) + dst);
            lds_copy16(reinterpret_cast<const uint8_t*>(gamma), cc * 4u,
                       lds_addr(g_lds) + (uint32_t)((k * 2 * 256) + wave * 64) * 16u);
            lds_copy16(reinterpret_cast<const uint8_t*>(gamma), cc * 4u + 16u,
                       lds_addr(g_lds) + (uint32_t)((k * 2 + 1) * 256 + wave * 64) * 16u);
        }
    } else {
        // the packed row: thread t's 16-byte pieces at 4096 k + 16 t, and the
        // row's scales (wave 0; lanes past KB repeat the last)
        const int arow = row_index ? row_index[0] : 0;
        const uint8_t* ac = act_codes + (size_t)arow * (size_t)H;
        for (int k = 0; k * 4096 < H; ++k)
            if (k * 4096 + t * 16 < H)
                lds_copy16(ac, (uint32_t)(k * 4096 + t * 16), lds_addr(a_lds) + (uint32_t)(k * 256 + wave * 64) * 16u);
        if (wave == 0)
            lds_copy4(act_scales + (size_t)arow * KB, (uint32_t)min(lane, KB - 1) * 4u, lds_addr(sa_lds));
    }
    // weight-scale rows: tile b + i*G lies in row ((b + i*G) * 16) >> 7;
    // slot i holds tile i's row (the host keeps ntiles <= kTail1MaxTiles)
    for (int i = wave; i < ntiles; i += 4)
        lds_copy4(w_scales + (size_t)(((b + i * G) * 16) >> 7) * KB, (uint32_t)min(lane, KB - 1) * 4u,
                  lds_addr(&sw_lds[0][0]) + (uint32_t)i * kStreamMaxKB * 4u);
    int rq = 0;   // next unit to request
#pragma unroll
    for (int s2 = 0; s2 < D - 1; ++s2) refill(s2, rq++);

    // 2. wait for this wave's norm (or packed-row) copies only (the sw rows
    //    and the ring stay in flight), then all waves' (barrier), then
    //    norm_quant_kernel's body
    {
        const int nsw = (ntiles - wave + 3) / 4;   // this wave's weight-scale copies
        wait_vm(max(nsw, 0) + (D - 1) * PER_BLOCK);
    }
    __syncthreads();
    float y[NSTEP][8];
    if (fused) {
    float sv[NSTEP][8];
    float4 graw[NSTEP][2];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const float live = k * 2048 + t * 8 < H ? 1.f : 0.f;
        const uint4 hv = h_lds[k * 256 + t], rv = r_lds[k * 256 + t];
        graw[k][0] = *reinterpret_cast<const float4*>(&g_lds[(k * 2) * 256 + t]);
        graw[k][1] = *reinterpret_cast<const float4*>(&g_lds[(k * 2 + 1) * 256 + t]);
        sv[k][0] = (bf16_lo(hv.x) + bf16_lo(rv.x)) * live;
        sv[k][1] = (bf16_hi(hv.x) + bf16_hi(rv.x)) * live;
        sv[k][2] = (bf16_lo(hv.y) + bf16_lo(rv.y)) * live;
        sv[k][3] = (bf16_hi(hv.y) + bf16_hi(rv.y)) * live;
        sv[k][4] = (bf16_lo(hv.z) + bf16_lo(rv.z)) * live;
        sv[k][5] = (bf16_hi(hv.z) + bf16_hi(rv.z)) * live;
        sv[k][6] = (bf16_lo(hv.w) + bf16_lo(rv.w)) * live;
        sv[k][7] = (bf16_hi(hv.w) + bf16_hi(rv.w)) * live;
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(sv[k][i], sv[k][i], ss);
    ss = wave_sum_f32(ss);
    if (lane == 0) wave_sum[wave] = ss;
    __syncthreads();
    const float total = (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
    const float rstd = (float)(1.0 / sqrt((double)total / (double)H + (double)eps));

    // every group computed (columns past H hold s = 0; they fill whole
    // 128-column blocks, which are not stored)
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const float4 g0 = graw[k][0], g1 = graw[k][1];
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[k][i] = (sv[k][i] * rstd) * g[i];
    }
    float bscale[NSTEP];
    uint2 code[NSTEP];
    quant_groups<NSTEP>(y, bscale, code);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
        const int c = k * 2048 + t * 8;
        if (c >= H) continue;   // uniform over each 16-thread scale block
        *reinterpret_cast<uint2*>(&a_lds[c]) = code[k];
        if ((t & 15) == 0) sa_lds[c >> 7] = bscale[k];
    }
    __syncthreads();
    }

    // 3. the weight stream: every unit's fragment rows all read the packed
    //    row; at each tile end the four partials meet in LDS (double-buffered
    //    by tile parity) and wave 0 folds the tile's keys into its running best
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    uint64_t best = 0;
    int ci = 0, cj = 0;   // unit being consumed: tile ci, slot cj
    // each unit's partial is promoted one unit late (pp, pf), beside the
    // next unit's MFMA; the order of the sum is unchanged
    v4f pp = v4f{0.f, 0.f, 0.f, 0.f};
    float pf = 0.f;
    auto compute = [&](int slot) {
        const bool live = ci < ntiles && cj < nb;
        const int kb = kb0 + max(min(cj, nb - 1), 0);
        const float swv = sw_lds[min(ci, ntiles - 1)][kb];
        const float f = sa_lds[kb] * (live ? swv : 0.f);
        const uint4 a0 = *reinterpret_cast<const uint4*>(&a_lds[kb * kBlock + fg * 16]);
        const uint4 a1 = *reinterpret_cast<const uint4*>(&a_lds[kb * kBlock + 64 + fg * 16]);
        const uint4* tw = &ring[wave][slot * SLOT];
        const v4f p = mfma_e4m3(make_frag(a0, a1), make_frag(tw[fpos0], tw[fpos1]));
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(pp[r], pf, acc[r]);
        pp = p;
        pf = f;
    };
    auto tile_end = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(pp[r], pf, acc[r]);   // the tile's last unit
        pf = 0.f;
        float* pb = &part[ci & 1][0][0];
        if (lane < 16) pb[wave * 16 + lane] = acc[0];
        acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
        __syncthreads();
        if (wave == 0 && lane < 16) {
            const float z = ((pb[lane] + pb[16 + lane]) + pb[32 + lane]) + pb[48 + lane];
            best = u64_max(best, argmax_key(z, (uint32_t)((b + ci * G) * 16 + lane)));
        }
    };
    for (int c = 0; c < nup; c += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            wait_vm((D - 2) * PER_BLOCK);
            refill((j + D - 1) % D, rq++);
            compute(j);
            if (ci < ntiles && cj == NBU - 1) tile_end();
            if (++cj == NBU) { cj = 0; ++ci; }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    MTPD_WAIT_VM(0);   // the clamped tail refills, before LDS is reused

    // 4. outputs of the row (workgroup 0), the row's best key, arrival
    if (fused && b == 0) {
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
            const int c = k * 2048 + t * 8;
            if (c < H) {
                *reinterpret_cast<uint4*>(out_hidden + c) = pack_bf16x8(y[k]);
                *reinterpret_cast<uint2*>(codes + c) = *reinterpret_cast<const uint2*>(&a_lds[c]);
            }
        }
        if (t < KB) scales[t] = sa_lds[t];
    }
    if (wave == 0) {
        best = row16_max_u64(best);
        uint64_t old = 0;
        if (lane == 0) old = merge_key(ws, 1, b, 0, best);
        const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
        if (lane == 0) last_flag = arrive_flat(ws, G, dep) ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<256>(ws, 1, out_max, out_idx, red);
}

bool use_draft_tail1(int64_t M, int64_t H) {
    if (plan_override().draft_tail_split) return false;   // norm_quant + LM head (testing)
    return M == 1 && H <= kTail1MaxH;
}

int64_t draft_tail1_grid(int64_t V) {
    // one resident workgroup per CU, at most kTail1MaxTiles tiles each
    const int64_t tiles = V / 16;
    return std::max<int64_t>(std::min<int64_t>(tiles, device_cus()), (tiles + kTail1MaxTiles - 1) / kTail1MaxTiles);
}

hipError_t launch_draft_tail1(const uint16_t* hidden, const uint16_t* residual, const float* gamma, float eps,
                              int64_t H, const uint8_t* w_codes, const float* w_scales, int64_t V,
                              uint16_t* out_hidden, uint8_t* codes, float* scales, float* out_max, int32_t* out_idx,
                              void* workspace, hipStream_t stream) {
    const int64_t tiles = V / 16;
    if (tiles > 0x7FFFFFFF || H > kTail1MaxH) return hipErrorInvalidValue;
    const int64_t grid = draft_tail1_grid(V);
    if (H <= 6144)
        hipLaunchKernelGGL(draft_tail1_kernel<3>, dim3((unsigned)grid), dim3(256), 0, stream, hidden, residual, gamma,
                           eps, (int)H, w_codes, w_scales, (int)tiles, out_hidden, codes, scales, out_max, out_idx,
                           argmax_ws(workspace, 1), nullptr, nullptr, nullptr);
    else
        hipLaunchKernelGGL(draft_tail1_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, hidden, residual, gamma,
                           eps, (int)H, w_codes, w_scales, (int)tiles, out_hidden, codes, scales, out_max, out_idx,
                           argmax_ws(workspace, 1), nullptr, nullptr, nullptr);
    return hipGetLastError();
}

bool use_lmhead1(const LmheadArgs& a) {
    // the persistent one-row kernel, unless a test pins another shape
    const PlanOverride& po = plan_override();
    return a.n_rows == 1 && a.H <= kTail1MaxH && po.lmhead_kernel == 0 && po.stream[0] == 0 &&
           !po.draft_tail_split;
}

hipError_t launch_lmhead1(const LmheadArgs& a, hipStream_t stream) {
    const int64_t tiles = a.V / 16;
    if (tiles > 0x7FFFFFFF || a.H > kTail1MaxH || a.n_rows != 1) return hipErrorInvalidValue;
    const int64_t grid = draft_tail1_grid(a.V);
    if (a.H <= 6144)
        hipLaunchKernelGGL(draft_tail1_kernel<3>, dim3((unsigned)grid), dim3(256), 0, stream, nullptr, nullptr, nullptr,
                           0.f, (int)a.H, a.w_codes, a.w_scales, (int)tiles, nullptr, nullptr, nullptr, a.out_max,
                           a.out_idx, argmax_ws(a.workspace, 1), a.a_codes, a.a_scales, a.row_index);
    else
        hipLaunchKernelGGL(draft_tail1_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, nullptr, nullptr, nullptr,
                           0.f, (int)a.H, a.w_codes, a.w_scales, (int)tiles, nullptr, nullptr, nullptr, a.out_max,
                           a.out_idx, argmax_ws(a.workspace, 1), a.a_codes, a.a_scales, a.row_index);
    return hipGetLastError();
}

#define MTPD_STREAM_CONFIGS(X) X(1, 1, 8) X(1, 1, 4) X(1, 1, 12) X(1, 2, 8) X(1, 2, 4) X(2, 1, 8) X(2, 2, 8)

bool stream_config_compiled(int nt, int ma, int d) {
#define MTPD_X(a, b, c) if (nt == a && ma == b && d == c) return true;
    MTPD_STREAM_CONFIGS(MTPD_X)
#undef MTPD_X
    return false;
}

int stream_max_h() { return kStreamMaxH; }

hipError_t launch_lmhead_stream(const LmheadArgs& a, int nt, int ma, int d, hipStream_t stream) {
    const int64_t tiles = a.V / (16 * nt);
    if (tiles > 0x7FFFFFFF || a.H > kStreamMaxH || a.n_rows > 8 * ma) return hipErrorInvalidValue;
#define MTPD_X(p, q, r)                                                                                   \
    if (nt == p && ma == q && d == r) {                                                                   \
        hipLaunchKernelGGL((lmhead_stream_kernel<p, q, r>), dim3((unsigned)tiles), dim3(64), 0, stream,   \
                           a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales,       \
                           (int)a.H, (int)tiles, a.out_max, a.out_idx, argmax_ws(a.workspace, a.n_rows)); \
        return hipGetLastError();                                                                         \
    }
    MTPD_STREAM_CONFIGS(MTPD_X)
#undef MTPD_X
    return hipErrorInvalidValue;
}

}  // namespace mtpd
