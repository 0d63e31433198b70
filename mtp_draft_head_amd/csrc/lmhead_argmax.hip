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

#include <stdio.h>
#include <algorithm>
#include <stdlib.h>
#include <string.h>

#include "kernels.h"
#include "lmhead_common.h"

namespace mtpd {

// f_lds[kb * ROWS + r] = sa[row r of the tile][kb] * sw[kb] for the tile's
// ROWS rows.  Loads are issued in batches with clamped (never branching)
// indices so each batch costs one memory latency; out-of-range slots are
// simply not stored.
template <bool GATHER, int ROWS, int NTHREADS>
__device__ __forceinline__ void stage_scales(float* f_lds, const float* __restrict__ a_scales,
                                             const int32_t* __restrict__ row_index,
                                             const float* __restrict__ swp, int m0, int n_rows, int KB) {
    const int n = KB * ROWS;
    constexpr int BATCH = 16;
    for (int base = 0; base < n; base += NTHREADS * BATCH) {
        float v[BATCH];
        int dst[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int e = base + i * NTHREADS + (int)threadIdx.x;
            const int ec = min(e, n - 1);
            const int r = ec / KB, kb = ec - r * KB;
            const int m = min(m0 + r, n_rows - 1);
            const int a = GATHER ? row_index[m] : m;
            v[i] = a_scales[(size_t)a * KB + kb] * swp[kb];
            dst[i] = e < n ? kb * ROWS + r : -1;
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            if (dst[i] >= 0) f_lds[dst[i]] = v[i];
    }
}

template <int MT, int NT, int S, int D>
__global__ __launch_bounds__(64 * S) void lmhead_argmax_kernel(
    const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales,
    const int32_t* __restrict__ row_index, int n_rows,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales, int H,
    int n_row_tiles, int total_tiles,
    float* __restrict__ out_max, int32_t* __restrict__ out_idx,
    ArgmaxWs ws)
{
    constexpr int ROWS = MT * 16;
    constexpr int COLS = NT * 16;
    extern __shared__ float lds[];
    __shared__ unsigned long long red[64 * S];
    __shared__ int last_flag;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
    const int KB = H >> 7;
    const int tile = xcd_contiguous((int)blockIdx.x, total_tiles);
    const int rt = tile % n_row_tiles;
    const int m0 = rt * ROWS;
    const int n0 = (tile / n_row_tiles) * COLS;
    const int vb = n0 >> 7;

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

    const int kb0 = (wave * KB) / S;
    const int kb1 = ((wave + 1) * KB) / S;

    // D-deep register ring: block kb+D is requested as soon as block kb has
    // been consumed, so D K blocks per wave are always in flight, and the
    // D blocks of one refill are consecutive 128-byte pieces of each row.
    // Only fragment loads sit in the vector-memory queue inside the loop (the
    // scales come from LDS), so each wait is for the oldest block alone.
    float acc[MT][NT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.f;

    v8i af[D][MT], wf[D][NT];
    float* f_lds = lds;   // [KB][ROWS]: sa[row][kb] * sw[vb][kb]
    auto load = [&](int j, int kb) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wf[j][nt] = load_frag(wp[nt] + kb * kBlock);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[j][mt] = load_frag(ap[mt] + kb * kBlock);
    };
    auto compute = [&](int j, int kb) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float4 f = *reinterpret_cast<const float4*>(&f_lds[kb * ROWS + mt * 16 + 4 * (lane >> 4)]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const v4f p = mfma_e4m3(af[j][mt], wf[j][nt]);
                acc[mt][nt][0] = fmaf(p[0], f.x, acc[mt][nt][0]);
                acc[mt][nt][1] = fmaf(p[1], f.y, acc[mt][nt][1]);
                acc[mt][nt][2] = fmaf(p[2], f.z, acc[mt][nt][2]);
                acc[mt][nt][3] = fmaf(p[3], f.w, acc[mt][nt][3]);
            }
        }
    };

    // Prologue: first the ring's first D blocks, then the combined scale
    // table of this row tile (sa * sw, K-major), whose loads overlap theirs.
    const bool ring = kb1 - kb0 >= D;
    if (ring) {
#pragma unroll
        for (int j = 0; j < D; ++j) load(j, kb0 + j);
    }
    {
        const float* swp = w_scales + (size_t)vb * KB;
        if (row_index)
            stage_scales<true, ROWS, 64 * S>(f_lds, a_scales, row_index, swp, m0, n_rows, KB);
        else
            stage_scales<false, ROWS, 64 * S>(f_lds, a_scales, row_index, swp, m0, n_rows, KB);
    }
    __syncthreads();

    int kb = kb0;
    if (ring) {
        for (; kb + 2 * D <= kb1; kb += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                compute(j, kb + j);
                load(j, kb + D + j);
                // keep the consume/refill order: without this the scheduler
                // hoists all D MFMAs above the refills and waits for the whole
                // ring at once
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < D; ++j) compute(j, kb + j);
        kb += D;
    }
    // fewer than D blocks left: request them all (indices clamped, so the
    // requests are unconditional), then consume the valid ones
    const int rem = kb1 - kb;
    if (rem > 0) {
#pragma unroll
        for (int j = 0; j < D - 1; ++j) load(j, min(kb + j, kb1 - 1));
#pragma unroll
        for (int j = 0; j < D - 1; ++j)
            if (j < rem) compute(j, kb + j);
    }

    if constexpr (S > 1) {
        float* part = lds + KB * ROWS;   // [(S-1)][MT*NT*4][64], after the scale table
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
        if (wave == 0) {
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
    }

    // wave 0: per-row best key of this tile (16-lane shuffle reduction over
    // the tile's columns), then one merge per row and the arrival.
    if (wave == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint64_t best = 0;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    best = u64_max(best, argmax_key(acc[mt][nt][i], (uint32_t)(n0 + nt * 16 + (lane & 15))));
                best = row16_max_u64(best);
                if ((lane & 15) == 0) red[mt * 16 + 4 * (lane >> 4) + i] = best;
            }
        }
        // ROWS <= 64: lane r merges row m0 + r
        uint64_t old = 0;
        if (lane < ROWS && m0 + lane < n_rows) old = merge_key(ws, n_rows, tile, m0 + lane, red[lane]);
        const unsigned int dep = __builtin_amdgcn_ballot_w64(never_nonzero(old) != 0) != 0 ? 1u : 0u;
        bool last = false;
        if (lane == 0) last = arrive(ws, tile, total_tiles, dep);
        if (lane == 0) last_flag = last ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;
    finalize_argmax<64 * S>(ws, n_rows, out_max, out_idx, red);
}

int device_cus() {
    // the override sizes the persistent grids as if the device had that many
    // CUs (testing: several tiles per workgroup at small vocab sizes)
    if (plan_override().device_cus > 0) return plan_override().device_cus;
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

namespace {

struct Tile {
    int mt, nt, s, d;
};

// (MT row tiles, NT column tiles per wave, S split-K waves, D ring depth)
// combinations compiled into the library.
#define MTPD_LM_CONFIGS(X)                                                                       \
    X(1, 1, 1, 8) X(1, 1, 2, 8) X(1, 1, 3, 8) X(1, 1, 4, 8) X(1, 1, 6, 8) X(1, 1, 8, 8)          \
    X(1, 1, 1, 4) X(1, 1, 2, 4) X(1, 1, 3, 4) X(1, 1, 4, 4) X(1, 1, 6, 4) X(1, 1, 8, 4)          \
    X(1, 2, 1, 4) X(1, 2, 2, 4) X(1, 2, 3, 4) X(1, 2, 4, 4) X(1, 2, 6, 4) X(1, 2, 8, 4)          \
    X(2, 2, 1, 4) X(2, 2, 2, 4) X(2, 2, 4, 4) X(2, 4, 1, 2) X(2, 4, 2, 2) X(2, 4, 4, 2)          \
    X(4, 2, 1, 2) X(4, 2, 2, 2) X(4, 2, 4, 2) X(4, 4, 1, 2) X(4, 4, 2, 2) X(4, 4, 4, 2)

bool compiled(const Tile& t) {
#define MTPD_X(a, b, c, e) if (t.mt == a && t.nt == b && t.s == c && t.d == e) return true;
    MTPD_LM_CONFIGS(MTPD_X)
#undef MTPD_X
    return false;
}


size_t lds_bytes(const Tile& t, int KB) {
    return (size_t)KB * t.mt * 16 * 4 + (size_t)(t.s - 1) * t.mt * t.nt * 4 * 64 * 4;
}

Tile choose_tile(int64_t n_rows, int64_t V, int64_t H) {
    const int KB = (int)(H / kBlock);
    Tile t;
    t.mt = n_rows <= 16 ? 1 : (n_rows <= 32 ? 2 : 4);
    t.nt = t.mt == 1 ? 1 : (t.mt == 2 ? 2 : 4);
    t.d = t.mt == 1 ? 8 : (t.mt == 2 ? 4 : 2);
    const int64_t row_tiles = (n_rows + t.mt * 16 - 1) / (t.mt * 16);
    const int64_t tiles = row_tiles * (V / (t.nt * 16));
    const int64_t want_waves = 8LL * device_cus();
    // split K across waves only when there are too few tiles to keep every CU
    // streaming (measured on the 1-row, 18944-row shard: 1184 single-wave
    // tiles, unsplit, beat any split)
    t.s = 1;
    if (t.mt == 1) t.d = 4;
    while (t.s < 4 && tiles * t.s < want_waves / 4 && 2 * t.s * t.d <= KB) t.s *= 2;
    // optional launch-shape override (tuning sweeps, tests)
    if (const int* o = plan_override().tile; o[0] > 0) {
        const Tile ot{t.mt, o[0], o[1], o[2]};
        if (compiled(ot)) t = ot;
    }
    while (!compiled(t) || lds_bytes(t, KB) > 64 * 1024) {
        if (t.s > 1) t.s /= 2;
        else if (t.d > 2) t.d /= 2;
        else break;
    }
    return t;
}

template <int MT, int NT, int S, int D>
hipError_t launch_t(const LmheadArgs& a, hipStream_t stream) {
    const int KB = (int)(a.H / kBlock);
    const int64_t row_tiles = (a.n_rows + MT * 16 - 1) / (MT * 16);
    const int64_t tiles = row_tiles * (a.V / (NT * 16));
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = lds_bytes(Tile{MT, NT, S, D}, KB);
    hipLaunchKernelGGL((lmhead_argmax_kernel<MT, NT, S, D>), dim3((unsigned)tiles), dim3(64 * S), lds, stream,
                       a.a_codes, a.a_scales, a.row_index, (int)a.n_rows, a.w_codes, a.w_scales, (int)a.H,
                       (int)row_tiles, (int)tiles, a.out_max, a.out_idx, argmax_ws(a.workspace, a.n_rows));
    return hipGetLastError();
}

}  // namespace

namespace {

struct DecodeTile {
    int mt, nt, d;
};

// The decode kernel serves n_rows <= 64 when a compiled (MT, NT, D) fits:
// D must divide H/128, 64*NT must divide V, and the LDS budget is 64 KB.
bool choose_decode(int64_t n_rows, int64_t V, int64_t H, DecodeTile* out) {
    // up to 16 rows the activation is small enough that single-wave tiles of
    // the generic kernel stream the weight faster than the LDS-sharing workgroups
    if (n_rows > 64 || n_rows <= 16) return false;
    const int KB = (int)(H / kBlock);
    const int mt = n_rows <= 16 ? 1 : (n_rows <= 32 ? 2 : 4);
    DecodeTile cand[6];
    int nc = 0;
    if (const int* o = plan_override().decode; o[0] > 0) cand[nc++] = DecodeTile{mt, o[0], o[1]};   // tuning
    if (mt == 1) {
        cand[nc++] = {1, 1, 8};
        cand[nc++] = {1, 1, 4};
    } else if (mt == 2) {
        cand[nc++] = {2, 1, 4};
        cand[nc++] = {2, 2, 4};
    } else {
        cand[nc++] = {4, 2, 2};
        cand[nc++] = {4, 1, 4};
    }
    for (int i = 0; i < nc; ++i) {
        const DecodeTile& c = cand[i];
        if (!decode_config_compiled(c.mt, c.nt, c.d)) continue;
        if (KB % c.d || V % (64 * c.nt)) continue;
        if (decode_config_lds(c.mt, c.d, KB) > 64 * 1024) continue;
        *out = c;
        return true;
    }
    return false;
}

}  // namespace

struct StreamTile {
    int nt, ma, d;
};

// Up to 16 rows and H <= stream_max_h(): the weight-streaming kernel, if a
// compiled (NT, MA, D) fits (16*NT must divide V; MA eight-row activation
// pieces; activation offsets are 32-bit).  The plan override's stream shape
// replaces NT and D (tuning).
bool use_stream(int64_t n_rows, int64_t V, int64_t H, int64_t a_rows, StreamTile* out) {
    if (plan_override().lmhead_kernel != 0) return false;
    if (n_rows < 1 || n_rows > 16 || H > stream_max_h() || a_rows * H > ((int64_t)1 << 32)) return false;
    const int ma = n_rows <= 8 ? 1 : 2;
    StreamTile cand[3];
    int nc = 0;
    if (const int* o = plan_override().stream; o[0] > 0) cand[nc++] = StreamTile{o[0], ma, o[1]};
    cand[nc++] = {1, ma, 8};
    cand[nc++] = {1, ma, 4};
    for (int i = 0; i < nc; ++i) {
        if (!stream_config_compiled(cand[i].nt, cand[i].ma, cand[i].d) || V % (16 * cand[i].nt)) continue;
        *out = cand[i];
        return true;
    }
    return false;
}

struct RowsTile {
    int mt, nt, nw, d;
    KouterTile ko;   // ko.tmax > 0: the K-outer kernel in that shape instead
};

// 17..64 rows, H <= stream_max_h(), 32-bit activation offsets: the streaming
// kernel with a shared activation ring, if a compiled (MT, NT, NW, D) fits
// (16*NT*NW must divide V).  The plan override's rows shape comes first (tuning).
bool use_rows(int64_t n_rows, int64_t V, int64_t H, int64_t a_rows, RowsTile* out) {
    if (plan_override().lmhead_kernel != 0) return false;
    if (n_rows <= 16 || n_rows > 64 || H > stream_max_h() || a_rows * H > ((int64_t)1 << 32)) return false;
    const int mt = n_rows <= 32 ? 2 : 4;
    RowsTile cand[4];
    int nc = 0;
    if (const int* o = plan_override().rows; o[0] > 0) cand[nc++] = RowsTile{mt, o[0], o[1], o[2], {}};
    if (mt == 4) {
        cand[nc++] = {4, 2, 4, 5};
        cand[nc++] = {4, 1, 4, 6};
    } else {
        cand[nc++] = {2, 2, 4, 4};
        cand[nc++] = {2, 1, 4, 6};
    }
    for (int i = 0; i < nc; ++i) {
        const RowsTile& c = cand[i];
        if (!rows_config_compiled(c.mt, c.nt, c.nw, c.d) || V % (16 * c.nt * c.nw)) continue;
        *out = c;
        // K outermost when every workgroup takes several tiles (the activation
        // is then copied once per workgroup, not once per tile)
        if (!kouter_choose(c.mt, V, device_cus(), &out->ko)) out->ko = KouterTile{0, 0, 0, 0};
        return true;
    }
    return false;
}

bool use_decode(int64_t n_rows, int64_t V, int64_t H, DecodeTile* dt) {
    // the override's "generic" forces the tiled kernel (testing)
    return plan_override().lmhead_kernel != 1 && choose_decode(n_rows, V, H, dt);
}

// many rows: the LDS-tiled 256 x 256 kernel
// The tiled kernel addresses the activation with 32-bit byte offsets.
bool use_gemm(int64_t n_rows, int64_t V, int64_t H, int64_t a_rows) {
    if (plan_override().lmhead_kernel == 1) return false;
    return n_rows > 64 && V % 256 == 0 && a_rows * H <= ((int64_t)1 << 32);
}

void describe_lmhead(int64_t n_rows, int64_t V, int64_t H, char* buf, size_t len) {
    DecodeTile dt;
    if (use_gemm(n_rows, V, H, n_rows)) {
        describe_gemm(n_rows, V, H, n_rows, buf, len);
        return;
    }
    {
        LmheadArgs a1{};
        a1.n_rows = n_rows;
        a1.a_rows = n_rows;
        a1.V = V;
        a1.H = H;
        if (use_lmhead1(a1)) {
            snprintf(buf, len, "draft_tail1_kernel (LM head only) grid=%lldx256 (%lld tiles)",
                     (long long)draft_tail1_grid(V), (long long)(V / 16));
            return;
        }
    }
    StreamTile st;
    if (use_stream(n_rows, V, H, n_rows, &st)) {
        snprintf(buf, len, "lmhead_stream_kernel<%d,%d,%d> grid=%lldx64", st.nt, st.ma, st.d,
                 (long long)(V / (16 * st.nt)));
        return;
    }
    RowsTile rt;
    if (use_rows(n_rows, V, H, n_rows, &rt)) {
        const long long tiles = (long long)(V / (16 * rt.nt * rt.nw));
        if (rt.ko.tmax > 0) {
            const long long kt = (long long)(V / (16 * rt.ko.nt * rt.ko.nw));
            snprintf(buf, len, "lmhead_kouter_kernel<%d,%d,%d,%d,%d> grid=%lldx%d (%lld tiles)", rt.mt, rt.ko.nt,
                     rt.ko.nw, rt.ko.d, rt.ko.tmax, std::min<long long>(kt, device_cus()), 64 * rt.ko.nw, kt);
            return;
        }
        const long long grid = std::max<long long>(std::min<long long>(tiles, device_cus()), (tiles + 15) / 16);
        snprintf(buf, len, "lmhead_stream_rows_kernel<%d,%d,%d,%d> grid=%lldx%d (%lld tiles)", rt.mt, rt.nt,
                 rt.nw, rt.d, grid, 64 * rt.nw, tiles);
        return;
    }
    if (use_decode(n_rows, V, H, &dt)) {
        snprintf(buf, len, "lmhead_decode_kernel<%d,%d,%d> grid=%lldx256", dt.mt, dt.nt, dt.d,
                 (long long)(V / (64 * dt.nt)));
        return;
    }
    const Tile t = choose_tile(n_rows, V, H);
    const long long tiles = (long long)((n_rows + t.mt * 16 - 1) / (t.mt * 16)) * (V / (t.nt * 16));
    snprintf(buf, len, "lmhead_argmax_kernel<%d,%d,%d,%d> grid=%lldx%d", t.mt, t.nt, t.s, t.d, tiles, 64 * t.s);
}

hipError_t launch_lmhead_argmax(const LmheadArgs& a, hipStream_t stream) {
    if (use_gemm(a.n_rows, a.V, a.H, a.a_rows)) return launch_lmhead_gemm(a, stream);
    if (use_lmhead1(a)) return launch_lmhead1(a, stream);
    StreamTile st;
    if (use_stream(a.n_rows, a.V, a.H, a.a_rows, &st)) return launch_lmhead_stream(a, st.nt, st.ma, st.d, stream);
    RowsTile rt;
    if (use_rows(a.n_rows, a.V, a.H, a.a_rows, &rt)) {
        if (rt.ko.tmax > 0)
            return launch_lmhead_kouter(a, rt.mt, rt.ko.nt, rt.ko.nw, rt.ko.d, rt.ko.tmax, device_cus(), stream);
        return launch_lmhead_rows(a, rt.mt, rt.nt, rt.nw, rt.d, device_cus(), stream);
    }
    DecodeTile dt;
    if (use_decode(a.n_rows, a.V, a.H, &dt))
        return launch_lmhead_decode(a, dt.mt, dt.nt, dt.d, stream);
    const Tile t = choose_tile(a.n_rows, a.V, a.H);
#define MTPD_X(p, q, r, u) \
    if (t.mt == p && t.nt == q && t.s == r && t.d == u) return launch_t<p, q, r, u>(a, stream);
    MTPD_LM_CONFIGS(MTPD_X)
#undef MTPD_X
    return hipErrorInvalidValue;
}

}  // namespace mtpd
