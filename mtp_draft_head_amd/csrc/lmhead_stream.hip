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
//    conflict-free (see ring_pos).
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
// LDS slot.  A fragment read has each group of 8 (or 16) consecutive lanes on
// 8 (16) consecutive rows and one K group: with s(r) = (r ^ (r >> 3)) & 7 the
// rows of such a group land on distinct 16-byte bank groups whether the LDS
// serves 128 or 256 bytes per cycle.
__device__ __forceinline__ int ring_pos(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

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
    // scales, copied once: sa_lds[r][kb] for fragment row r (rows past the
    // last activation row repeat it), sw_lds[kb] for the tiles' 128-row block;
    // entries past KB repeat the last block
    __shared__ __align__(16) float sa_lds[16 * kStreamMaxKB];
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
            for (int q = 0; q < 2; ++q) lds_copy16(wb, woff[nt][q], ring0 + (uint32_t)(j * SLOT + (nt * 2 + q) * 64) * 16u);
#pragma unroll
        for (int q = 0; q < MA; ++q) lds_copy16(ab, aoff[q], ring0 + (uint32_t)(j * SLOT + (NT * 2 + q) * 64) * 16u);
    };

    float acc[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] = 0.f;

    // scale reads: rows 4 * fg + i of block kb; padding blocks (kb >= KB) get
    // a zero factor
    const float* sar = &sa_lds[4 * fg * kStreamMaxKB];
    auto compute = [&](int j, int kb) {
        const int kc = min(kb, kStreamMaxKB - 1);
        const float swl = sw_lds[kc];
        const float sw = kb < KB ? swl : 0.f;
        const float4 f = make_float4(sar[kc] * sw, sar[kStreamMaxKB + kc] * sw, sar[2 * kStreamMaxKB + kc] * sw,
                                     sar[3 * kStreamMaxKB + kc] * sw);
        const uint4* ta = &ring[j * SLOT + NT * 128];
        const v8i af = make_frag(ta[apos0], ta[apos1]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint4* tw = &ring[j * SLOT + nt * 128];
            const v4f p = mfma_e4m3(af, make_frag(tw[fpos0], tw[fpos1]));
            acc[nt][0] = fmaf(p[0], f.x, acc[nt][0]);
            acc[nt][1] = fmaf(p[1], f.y, acc[nt][1]);
            acc[nt][2] = fmaf(p[2], f.z, acc[nt][2]);
            acc[nt][3] = fmaf(p[3], f.w, acc[nt][3]);
        }
    };

    // prologue: the scales (16 activation rows and the weight-scale row, 64
    // blocks each), then the first D ring blocks.  All are copies into LDS,
    // older than any ring block, so the first ring wait covers them.  The
    // gathered row numbers are loaded first and waited for here: a register
    // load completing after the copies were issued would make the compiler
    // wait for those too.
    uint32_t srow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int mr = min(r, n_rows - 1);
        srow[r] = (uint32_t)(row_index ? row_index[mr] : mr);
    }
    MTPD_WAIT_VM(0);
    asm volatile("" ::: "memory");
    {
        const uint32_t kl = (uint32_t)min(lane, KB - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            lds_copy4(a_scales, (srow[r] * (uint32_t)KB + kl) * 4u, lds_addr(&sa_lds[r * kStreamMaxKB]));
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

    // per activation row (4 * (lane / 16) + i) the best key over the wave's
    // NT * 16 vocab rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint64_t best = 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            best = u64_max(best, argmax_key(acc[nt][i], (uint32_t)(n0 + nt * 16 + (lane & 15))));
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) best = u64_max(best, shfl_xor_u64(best, off));
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
