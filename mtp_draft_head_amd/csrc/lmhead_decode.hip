// Block-scaled FP8 LM head + greedy argmax for the weight-streaming (decode)
// regime: at most 64 activation rows, so the cost is reading the weight once.
//
// Same result definition as lmhead_argmax.hip (packed activation consumed as
// is, "[Quant][MTP] Reuse packed FP8 logits inputs", Purpose and
// Dependencies; local argmax with the lowest index on equal logits, "[Spec
// Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax draft
// tokens", Summary).  What changes is the schedule:
//
//  - A workgroup is 4 waves over 4*NT*16 consecutive vocab rows and all
//    MT*16 activation rows; each wave owns NT 16-row weight tiles and walks
//    the whole K range, so every workgroup does the same amount of work and,
//    with at most a few hundred to a couple of thousand workgroups, all of
//    them are resident at once and finish together.
//  - Weight fragments go straight from HBM into a D-deep VGPR ring per wave
//    (each refill is 128 contiguous bytes per weight row).
//  - The packed activation is shared: per chunk of D K blocks the four waves
//    stage the chunk's activation fragments into LDS (double-buffered, one
//    barrier per chunk), laid out so each lane's 16-byte LDS read is
//    conflict-free; without this every wave would re-read the activation
//    from L2 and the activation traffic would match or exceed the weight's.
//  - Activation scales live in LDS (K-major), the wave's weight-scale row in
//    LDS too; the fp32 promotion is acc += p * (sa * sw) per K block.
//  - Epilogue: per-row best keys of the four waves meet in LDS, one merge per
//    row per workgroup into a partitioned key slot, then the two-level
//    arrival; the last workgroup decodes and clears the workspace.

#include "kernels.h"
#include "lmhead_common.h"

namespace mtpd {

template <int MT, int NT, int D>
__global__ __launch_bounds__(256) void lmhead_decode_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int total_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx,
    ArgmaxWs ws)
{
    constexpr int ROWS = MT * 16;
    constexpr int WCOLS = NT * 16;
    constexpr int COLS = 4 * WCOLS;
    constexpr int PIECES = D * MT * 2;        // 1 KB activation pieces per chunk
    constexpr int PPW = (PIECES + 3) / 4;     // pieces each wave stages

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ unsigned long long red[256];
    __shared__ int last_flag;

    const int KB = H >> 7;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform, in an SGPR
    const int tile = xcd_contiguous((int)blockIdx.x, total_tiles);
    const int n0 = tile * COLS + wave * WCOLS;      // this wave's first vocab row

    float* sa_lds = reinterpret_cast<float*>(smem);                    // [KB][ROWS]
    float* sw_lds = sa_lds + KB * ROWS;                                // [4][KB]
    uint4* abuf = reinterpret_cast<uint4*>(sw_lds + 4 * KB);           // [2][PIECES][64]

    // weight fragment pointers (row n0 + nt*16 + lane%16, K-byte (lane/16)*16)
    const uint8_t* wp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        wp[nt] = w_codes + (size_t)(n0 + nt * 16 + (lane & 15)) * H + (lane >> 4) * 16;

    // activation pieces this lane stages: piece p = wave + 4*i covers
    // (block j, row tile mt, half h) of a chunk
    const uint8_t* pp[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        const int p = min(wave + 4 * i, PIECES - 1);
        const int j = p / (MT * 2), mt = (p >> 1) % MT, h = p & 1;
        const int m = min(mt * 16 + (lane & 15), n_rows - 1);
        const int a = row_index ? row_index[m] : m;
        pp[i] = a_codes + (size_t)a * H + (lane >> 4) * 16 + j * kBlock + h * 64;
    }

    float acc[MT][NT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.f;

    v8i wf[D][NT];
    // a native vector type: a uint4 struct temporary would be folded into a
    // global-to-LDS memcpy placed at the store, i.e. a late load
    u32x4 areg[PPW];
    // pieces beyond PIECES (PIECES not a multiple of 4) are loaded but never stored
#define MTPD_LOAD_A(chunk)                                                                 \
    _Pragma("unroll") for (int i = 0; i < PPW; ++i)                                        \
        areg[i] = *reinterpret_cast<const u32x4*>(pp[i] + (chunk) * (D * kBlock));
#define MTPD_STORE_A(buf)                                                                  \
    _Pragma("unroll") for (int i = 0; i < PPW; ++i)                                        \
        if (PIECES % 4 == 0 || wave + 4 * i < PIECES)                                      \
            *reinterpret_cast<u32x4*>(&abuf[((buf) * PIECES + wave + 4 * i) * 64 + lane]) = areg[i];
    auto load_w = [&](int j, int kb) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wf[j][nt] = load_frag(wp[nt] + kb * kBlock);
    };
    auto compute = [&](int buf, int j, int kb) {
        const float sw = sw_lds[wave * KB + kb];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int p0 = (j * MT + mt) * 2;
            const v8i af = make_frag(abuf[(buf * PIECES + p0) * 64 + lane], abuf[(buf * PIECES + p0 + 1) * 64 + lane]);
            const float4 sa = *reinterpret_cast<const float4*>(&sa_lds[kb * ROWS + mt * 16 + 4 * (lane >> 4)]);
            const float f0 = sa.x * sw, f1 = sa.y * sw, f2 = sa.z * sw, f3 = sa.w * sw;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const v4f p = mfma_e4m3(af, wf[j][nt]);
                acc[mt][nt][0] = fmaf(p[0], f0, acc[mt][nt][0]);
                acc[mt][nt][1] = fmaf(p[1], f1, acc[mt][nt][1]);
                acc[mt][nt][2] = fmaf(p[2], f2, acc[mt][nt][2]);
                acc[mt][nt][3] = fmaf(p[3], f3, acc[mt][nt][3]);
            }
        }
    };

    // Prologue: weight ring for chunk 0, activation chunk 0, then the scale
    // tables (their loads overlap the ring's).
#pragma unroll
    for (int j = 0; j < D; ++j) load_w(j, j);
    MTPD_LOAD_A(0)
    {
        const int n = KB * ROWS;
        for (int base = 0; base < n; base += 256 * 8) {
            float v[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + u * 256 + t;
                const int ec = min(e, n - 1);
                const int r = ec / KB, kb = ec - r * KB;
                const int m = min(r, n_rows - 1);
                const int a = row_index ? row_index[m] : m;
                v[u] = a_scales[(size_t)a * KB + kb];
                dst[u] = e < n ? kb * ROWS + r : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (dst[u] >= 0) sa_lds[dst[u]] = v[u];
        }
        // weight-scale row of each wave's 128-row block
        for (int e = t; e < 4 * KB; e += 256) {
            const int w = e / KB, kb = e - w * KB;
            sw_lds[e] = w_scales[(size_t)((tile * COLS + w * WCOLS) >> 7) * KB + kb];
        }
    }
    MTPD_STORE_A(0)
    __syncthreads();

    const int nchunks = KB / D;
    // one chunk: consume ring slot j (block c*D + j) and refill it with block
    // (c+1)*D + j; the activation for chunk c+1 is fetched at the start and
    // parked in LDS at the end
    for (int c = 0; c + 1 < nchunks; ++c) {
        const int buf = c & 1;
        MTPD_LOAD_A(c + 1)
        // issue the activation fetch here, ahead of the chunk's weight refills:
        // IR-level sinking would otherwise move it next to its LDS store, and
        // the in-order vmcnt wait there would drain the whole weight ring
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < D; ++j) {
            compute(buf, j, c * D + j);
            load_w(j, (c + 1) * D + j);
            __builtin_amdgcn_sched_barrier(0);
        }
        MTPD_STORE_A(buf ^ 1)
        __syncthreads();
    }
    {
        const int c = nchunks - 1;
#pragma unroll
        for (int j = 0; j < D; ++j) compute(c & 1, j, c * D + j);
    }

    // per-row best over this wave's columns, then over the four waves
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint64_t best = 0;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                best = u64_max(best, argmax_key(acc[mt][nt][i], (uint32_t)(n0 + nt * 16 + (lane & 15))));
            best = row16_max_u64(best);
            if ((lane & 15) == 0) red[wave * ROWS + mt * 16 + 4 * (lane >> 4) + i] = best;
        }
    }
    __syncthreads();
    if (wave == 0) {
        uint64_t old = 0;
        if (lane < ROWS && lane < n_rows) {
            const uint64_t k = u64_max(u64_max(red[lane], red[ROWS + lane]),
                                       u64_max(red[2 * ROWS + lane], red[3 * ROWS + lane]));
            old = merge_key(ws, n_rows, tile, lane, k);
        }
        const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
        bool last = false;
        if (lane == 0) last = arrive(ws, tile, total_tiles, dep);
        if (lane == 0) last_flag = last ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<256>(ws, n_rows, out_max, out_idx, red);
#undef MTPD_LOAD_A
#undef MTPD_STORE_A
}

namespace {

size_t decode_lds_bytes(int MT, int D, int KB) {
    return (size_t)KB * MT * 16 * 4 + (size_t)4 * KB * 4 + (size_t)2 * D * MT * 2 * 1024;
}

template <int MT, int NT, int D>
hipError_t launch_decode_t(const LmheadArgs& a, hipStream_t stream) {
    const int KB = (int)(a.H / kBlock);
    const int64_t tiles = a.V / (4 * NT * 16);
    hipLaunchKernelGGL((lmhead_decode_kernel<MT, NT, D>), dim3((unsigned)tiles), dim3(256),
                       decode_lds_bytes(MT, D, KB), stream, a.a_codes, a.a_scales, a.row_index, (int)a.n_rows,
                       a.w_codes, a.w_scales, (int)a.H, (int)tiles, a.out_max, a.out_idx,
                       argmax_ws(a.workspace, a.n_rows));
    return hipGetLastError();
}

}  // namespace

// (MT, NT, D) combinations compiled for the decode kernel.
#define MTPD_DECODE_CONFIGS(X) \
    X(1, 1, 8) X(1, 1, 4) X(1, 2, 4) X(1, 2, 8) X(2, 1, 4) X(2, 2, 4) X(4, 2, 2) X(4, 4, 2) X(4, 2, 4) X(4, 1, 4)

bool decode_config_compiled(int mt, int nt, int d) {
#define MTPD_X(p, q, r) if (mt == p && nt == q && d == r) return true;
    MTPD_DECODE_CONFIGS(MTPD_X)
#undef MTPD_X
    return false;
}

size_t decode_config_lds(int mt, int d, int KB) { return decode_lds_bytes(mt, d, KB); }

hipError_t launch_lmhead_decode(const LmheadArgs& a, int mt, int nt, int d, hipStream_t stream) {
#define MTPD_X(p, q, r) if (mt == p && nt == q && d == r) return launch_decode_t<p, q, r>(a, stream);
    MTPD_DECODE_CONFIGS(MTPD_X)
#undef MTPD_X
    return hipErrorInvalidValue;
}

}  // namespace mtpd
