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

struct LmheadArgs {
    const uint8_t* a_codes;
    const float* a_scales;
    const int32_t* row_index;   // NULL: identity
    int64_t n_rows;
    const uint8_t* w_codes;
    const float* w_scales;
    int64_t V;
    int64_t H;
    float* out_max;
    int32_t* out_idx;
    void* workspace;            // [n_rows] u64 keys, then a u32 completion counter
};

hipError_t launch_lmhead_argmax(const LmheadArgs& a, hipStream_t stream);

// Workspace layout shared by the launcher and the C ABI.
inline size_t workspace_bytes(int64_t n_rows) {
    if (n_rows <= 0) return 0;
    const size_t raw = (size_t)n_rows * 8 + 8;
    return (raw + 255) & ~(size_t)255;
}

}  // namespace mtpd
