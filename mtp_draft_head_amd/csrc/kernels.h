// Launchers of the gfx950 kernels (host side).  Arguments are validated by
// the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtpd {

constexpr int kBlock = 128;   // scale-block width along K (and along V for the weight)

hipError_t launch_norm_quant(const uint16_t* hidden, const uint16_t* residual, const float* gamma,
                             float eps, int64_t M, int64_t H, uint16_t* out_hidden, uint8_t* codes,
                             float* scales, hipStream_t stream);

// Row-parallel partial outputs summed by allreduce_norm_quant_kernel: n
// device pointers, each [M][H] bf16 (passed by value as a kernel argument).
constexpr int kMaxPartials = 16;
struct PartialPtrs {
    const uint16_t* p[kMaxPartials];
    int n;
};

hipError_t launch_allreduce_norm_quant(const PartialPtrs& parts, const uint16_t* residual, const float* gamma,
                                       float eps, int64_t M, int64_t H, uint16_t* out_hidden, uint8_t* codes,
                                       float* scales, hipStream_t stream);

// Vocab-parallel combine of per-shard (max, local index) pairs
// (argmax_combine.hip): offsets by value, at most kMaxShards shards.
constexpr int kMaxShards = 64;
struct ShardOffsets {
    uint32_t off[kMaxShards];
};

hipError_t launch_argmax_combine(const float* local_max, const int32_t* local_idx, const ShardOffsets& offs,
                                 int n_shards, int64_t n_rows, float* out_max, int32_t* out_idx,
                                 hipStream_t stream);
// top-k lists of at most kMaxTopk keys per row and shard (argmax_combine.hip)
constexpr int kMaxTopk = 32;
hipError_t launch_topk_combine(const float* local_val, const int32_t* local_idx, const ShardOffsets& offs,
                               int n_shards, int64_t n_rows, int k, float* out_val, int32_t* out_idx,
                               hipStream_t stream);

struct LmheadArgs {
    const uint8_t* a_codes;
    const float* a_scales;
    const int32_t* row_index;   // NULL: identity
    int64_t n_rows;
    int64_t a_rows;             // rows of the packed activation (row_index values lie below)
    const uint8_t* w_codes;
    const float* w_scales;
    int64_t V;
    int64_t H;
    float* out_max;
    int32_t* out_idx;
    void* workspace;            // layout below
};

hipError_t launch_lmhead_argmax(const LmheadArgs& a, hipStream_t stream);

// one packed row: the persistent one-row kernel of the fused tail as the LM
// head alone
bool use_lmhead1(const LmheadArgs& a);
hipError_t launch_lmhead1(const LmheadArgs& a, hipStream_t stream);

// name and launch shape of the kernel launch_lmhead_argmax picks
void describe_lmhead(int64_t n_rows, int64_t V, int64_t H, char* buf, size_t len);

// the compute-regime kernels (lmhead_gemm.hip): 256-column tiles, V % 256 == 0
hipError_t launch_lmhead_gemm(const LmheadArgs& a, hipStream_t stream);
void describe_gemm(int64_t n_rows, int64_t V, int64_t H, int64_t a_rows, char* buf, size_t len);

// the weight-streaming kernel for one row tile (lmhead_stream.hip): n_rows <= 16
bool stream_config_compiled(int nt, int ma, int d);
int stream_max_h();
hipError_t launch_lmhead_stream(const LmheadArgs& a, int nt, int ma, int d, hipStream_t stream);

// the weight-streaming kernel with a shared activation ring (lmhead_stream.hip): n_rows <= 64
bool rows_config_compiled(int mt, int nt, int nw, int d);
hipError_t launch_lmhead_rows(const LmheadArgs& a, int mt, int nt, int nw, int d, int cus, hipStream_t stream);
// the same rows with K outermost and each workgroup's tmax tiles inner
// (lmhead_stream.hip): a compiled shape for mt row tiles and V on cus CUs,
// used when every workgroup takes at least two tiles
struct KouterTile {
    int nt, nw, d, tmax;
};
bool kouter_choose(int mt, int64_t V, int cus, KouterTile* out);
hipError_t launch_lmhead_kouter(const LmheadArgs& a, int mt, int nt, int nw, int d, int tmax, int cus,
                                hipStream_t stream);

// multiprocessor count of the current device (cached per device), or the
// plan override's count
int device_cus();

// Launch-plan overrides for tuning sweeps and tests, written only by
// mtpd_set_plan_override (all zero: the dispatcher chooses).  Process-wide;
// read by the host-side dispatch of every call.
struct PlanOverride {
    int lmhead_kernel;       // 0 auto; 1 the generic tiled kernel only; 2 no streaming kernels (decode or generic)
    int tile[3];             // generic kernel nt, s, d
    int stream[2];           // weight-streaming kernel nt, d
    int rows[3];             // shared-activation streaming kernel nt, nw, d
    int decode[2];           // register-staged decode kernel nt, d
    int kouter;              // 0 auto; -1 never; 1 only the shape in kouter_shape
    int kouter_shape[4];     // nt, nw, d, tmax
    int draft_tail_split;    // 1: one row runs norm_quant + the LM head, not the fused tail
    int device_cus;          // > 0: persistent grids sized as if the device had this many CUs
    int gemm;                // 0 auto; otherwise a compute-regime kernel variant (lmhead_gemm.hip)
    int norm_quant;          // 0 a workgroup per row; 1 a wavefront per row (H <= 8192)
};
const PlanOverride& plan_override();

// top-k of the LM head (lmhead_stream.hip): at most 64 rows per call, k <= 32;
// workspace: the candidate lists (no zeroing needed)
bool topk_supported(int64_t H, int64_t a_rows);
size_t topk_workspace_bytes(int64_t n_rows, int64_t V, int64_t k);
hipError_t launch_lmhead_topk(const LmheadArgs& a, int k, float* out_val, int32_t* out_idx, int cus,
                              hipStream_t stream);

// the fused one-row draft tail (lmhead_stream.hip): M == 1, H <= 8192
bool use_draft_tail1(int64_t M, int64_t H);
int64_t draft_tail1_grid(int64_t V);   // workgroups of the fused one-row launch
hipError_t launch_draft_tail1(const uint16_t* hidden, const uint16_t* residual, const float* gamma, float eps,
                              int64_t H, const uint8_t* w_codes, const float* w_scales, int64_t V,
                              uint16_t* out_hidden, uint8_t* codes, float* scales, float* out_max, int32_t* out_idx,
                              void* workspace, hipStream_t stream);

// the decode-regime kernel (lmhead_decode.hip): n_rows <= 64
bool decode_config_compiled(int mt, int nt, int d);
size_t decode_config_lds(int mt, int d, int KB);
hipError_t launch_lmhead_decode(const LmheadArgs& a, int mt, int nt, int d, hipStream_t stream);

// Workspace of the LM-head kernels (all of it zero between calls):
//   keys      P partitions x n_rows u64 argmax keys.  While P * n_rows <= 4096
//             every key sits on its own 128-byte line (stride 16 u64), so
//             workgroups merging into different slots never share a line;
//             beyond that (large n_rows, P = 1) keys are dense.
//   counters  33 u32 arrival counters, one per 128-byte line (32 groups +
//             the top), after the keys padded to 256 bytes.
constexpr int kArriveGroups = 32;

inline int workspace_partitions(int64_t n_rows) {
    int P = 256;
    while (P > 1 && n_rows > 4096 / P) P >>= 1;   // P * n_rows > 4096, without overflow
    return P;
}

inline int workspace_key_stride(int64_t n_rows) {
    return n_rows <= 4096 / workspace_partitions(n_rows) ? 16 : 1;
}

inline size_t workspace_key_bytes(int64_t n_rows) {
    const size_t raw =
        (size_t)workspace_partitions(n_rows) * (size_t)n_rows * (size_t)workspace_key_stride(n_rows) * 8;
    return (raw + 255) & ~(size_t)255;
}

inline size_t workspace_bytes(int64_t n_rows) {
    if (n_rows <= 0) return 0;
    return workspace_key_bytes(n_rows) + (size_t)(kArriveGroups + 1) * 128 + 128;   // padded to 256
}

}  // namespace mtpd
