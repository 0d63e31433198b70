// C ABI of libmtpd: argument validation, error reporting and dispatch.
// Every argument is checked before the first HIP call, so an invalid call
// launches nothing and touches no device state.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kernels.h"
#include "mtpd.h"

namespace {

thread_local char g_err[512] = {0};

mtpd_status fail(mtpd_status st, const char* fmt, ...) {
    if (g_err[0] == 0) {   // the first failure is the root cause; keep it
        int n = snprintf(g_err, sizeof g_err, "%s: ", mtpd_status_name(st));
        if (n < 0) n = 0;
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(g_err + n, sizeof g_err - (size_t)n, fmt, ap);
        va_end(ap);
    }
    return st;
}

constexpr int64_t kMaxH = 16384;
constexpr int64_t kMaxV = 0x7FFFFF80LL;   // 2^31 - 128
constexpr int64_t kMaxRows = 1LL << 24;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
    const void* p;
    size_t bytes;
    const char* name;
};

bool overlap(const Range& a, const Range& b) {
    if (!a.bytes || !b.bytes) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// outputs must not overlap each other nor any input
mtpd_status check_alias(const Range* outs, int n_out, const Range* ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(MTPD_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j]))
                return fail(MTPD_ERR_ALIAS, "%s overlaps input %s", outs[i].name, ins[j].name);
    }
    return MTPD_OK;
}

mtpd_status check_H(int64_t H) {
    if (H < mtpd::kBlock || H > kMaxH || H % mtpd::kBlock)
        return fail(MTPD_ERR_SHAPE, "H=%lld must be a multiple of 128 in [128, %lld]", (long long)H,
                    (long long)kMaxH);
    return MTPD_OK;
}

mtpd_status check_weight(const mtpd_fp8_weight* w, int64_t H) {
    if (!w) return fail(MTPD_ERR_NULL, "weight descriptor is NULL");
    if (!w->codes || !w->scales) return fail(MTPD_ERR_NULL, "weight codes/scales pointer is NULL");
    if (w->H != H) return fail(MTPD_ERR_SHAPE, "weight H=%lld differs from H=%lld", (long long)w->H, (long long)H);
    if (w->V < mtpd::kBlock || w->V > kMaxV || w->V % mtpd::kBlock)
        return fail(MTPD_ERR_SHAPE, "V=%lld must be a multiple of 128 in [128, 2^31-128]", (long long)w->V);
    if (!aligned(w->codes, 16)) return fail(MTPD_ERR_ALIGN, "weight codes not 16-byte aligned");
    if (!aligned(w->scales, 4)) return fail(MTPD_ERR_ALIGN, "weight scales not 4-byte aligned");
    return MTPD_OK;
}

mtpd_status check_norm_args(const uint16_t* hidden, const uint16_t* residual, const float* norm_weight,
                            int64_t M, int64_t H, const uint16_t* out_hidden, const mtpd_qact* out_act) {
    if (M < 0 || M > kMaxRows) return fail(MTPD_ERR_SHAPE, "M=%lld out of [0, 2^24]", (long long)M);
    mtpd_status st = check_H(H);
    if (st != MTPD_OK) return st;
    if (!out_act) return fail(MTPD_ERR_NULL, "out_act descriptor is NULL");
    if (out_act->rows != M || out_act->cols != H)
        return fail(MTPD_ERR_SHAPE, "out_act is [%lld x %lld], expected [%lld x %lld]", (long long)out_act->rows,
                    (long long)out_act->cols, (long long)M, (long long)H);
    if (M == 0) return MTPD_OK;
    if (!hidden || !residual || !norm_weight || !out_hidden || !out_act->codes || !out_act->scales)
        return fail(MTPD_ERR_NULL, "a required pointer is NULL");
    if (!aligned(hidden, 16) || !aligned(residual, 16) || !aligned(out_hidden, 16) ||
        !aligned(out_act->codes, 16) || !aligned(norm_weight, 16))
        return fail(MTPD_ERR_ALIGN, "bf16/code/norm-weight arrays must be 16-byte aligned");
    if (!aligned(out_act->scales, 4)) return fail(MTPD_ERR_ALIGN, "scales not 4-byte aligned");
    return MTPD_OK;
}

mtpd_status check_lmhead_outputs(int64_t n_rows, const float* out_max, const int32_t* out_idx,
                                 const void* workspace, size_t workspace_bytes) {
    if (!out_max || !out_idx) return fail(MTPD_ERR_NULL, "out_max/out_idx is NULL");
    if (!aligned(out_max, 4) || !aligned(out_idx, 4)) return fail(MTPD_ERR_ALIGN, "out_max/out_idx not 4-byte aligned");
    const size_t need = mtpd::workspace_bytes(n_rows);
    if (!workspace || workspace_bytes < need)
        return fail(MTPD_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", workspace_bytes, workspace,
                    need);
    if (!aligned(workspace, 256)) return fail(MTPD_ERR_ALIGN, "workspace not 256-byte aligned");
    return MTPD_OK;
}

mtpd_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MTPD_OK;
    return fail(MTPD_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

mtpd::PlanOverride g_plan{};

// ---- scratch of the allocation-free entry point ----
// The argmax keys and arrival counters of mtpd_draft_tail_noalloc live in one
// file-scope device array (one copy per GPU, held until the process ends),
// sized for 65536 rows: the largest workspace_bytes(n) for n <= 65536 is
// 512 KiB of keys plus the counter lines.  Host code never uses the array's
// name as an address: each device's address comes from hipGetSymbolAddress.
constexpr int64_t kNoallocMaxRows = 65536;
constexpr size_t kScratchBytes = 524288 + (size_t)(mtpd::kArriveGroups + 1) * 128 + 128;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {nullptr};
bool g_scratch_zeroed[kMaxDevices] = {false};

__global__ void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// "a,b,c" -> n ints, all positive; false if it does not parse
bool parse_ints(const char* v, int* out, int n) {
    int got = 0;
    const char* p = v;
    while (got < n) {
        char* end = nullptr;
        const long x = strtol(p, &end, 10);
        if (end == p || x <= 0 || x > 1 << 20) return false;
        out[got++] = (int)x;
        if (got < n) {
            if (*end != ',') return false;
            p = end + 1;
        } else if (*end != 0) {
            return false;
        }
    }
    return true;
}

}  // namespace

namespace mtpd {
const PlanOverride& plan_override() { return g_plan; }
}  // namespace mtpd

extern "C" {

mtpd_status mtpd_set_plan_override(const char* key, const char* value) {
    if (!key) {
        g_plan = mtpd::PlanOverride{};
        return MTPD_OK;
    }
    mtpd::PlanOverride p = g_plan;
    const bool clear = value == nullptr;
    bool ok = true;
    if (!strcmp(key, "lmhead_kernel")) {
        if (clear) p.lmhead_kernel = 0;
        else if (!strcmp(value, "generic")) p.lmhead_kernel = 1;
        else if (!strcmp(value, "decode")) p.lmhead_kernel = 2;
        else ok = false;
    } else if (!strcmp(key, "lmhead_tile")) {
        int v[3] = {0, 0, 0};
        ok = clear || parse_ints(value, v, 3);
        memcpy(p.tile, v, sizeof v);
    } else if (!strcmp(key, "lmhead_stream")) {
        int v[2] = {0, 0};
        ok = clear || parse_ints(value, v, 2);
        memcpy(p.stream, v, sizeof v);
    } else if (!strcmp(key, "lmhead_rows")) {
        int v[3] = {0, 0, 0};
        ok = clear || parse_ints(value, v, 3);
        memcpy(p.rows, v, sizeof v);
    } else if (!strcmp(key, "lmhead_decode")) {
        int v[2] = {0, 0};
        ok = clear || parse_ints(value, v, 2);
        memcpy(p.decode, v, sizeof v);
    } else if (!strcmp(key, "lmhead_kouter")) {
        int v[4] = {0, 0, 0, 0};
        if (clear) p.kouter = 0;
        else if (!strcmp(value, "0")) p.kouter = -1;
        else if ((ok = parse_ints(value, v, 4))) p.kouter = 1;
        memcpy(p.kouter_shape, v, sizeof v);
    } else if (!strcmp(key, "lmhead_gemm")) {
        int v = 0;
        ok = clear || !strcmp(value, "0") || parse_ints(value, &v, 1);
        p.gemm = v;
    } else if (!strcmp(key, "draft_tail")) {
        ok = clear || !strcmp(value, "split");
        p.draft_tail_split = clear ? 0 : 1;
    } else if (!strcmp(key, "norm_quant")) {
        ok = clear || !strcmp(value, "wave") || !strcmp(value, "workgroup");
        p.norm_quant = !clear && !strcmp(value, "wave") ? 1 : 0;
    } else if (!strcmp(key, "device_cus")) {
        int v = 0;
        ok = clear || parse_ints(value, &v, 1);
        p.device_cus = v;
    } else {
        return fail(MTPD_ERR_SHAPE, "unknown plan-override key \"%s\"", key);
    }
    if (!ok) return fail(MTPD_ERR_SHAPE, "plan override %s: value \"%s\" does not parse", key, value);
    g_plan = p;
    return MTPD_OK;
}

const char* mtpd_status_name(mtpd_status s) {
    // A C caller may pass any int; in C++ loading an enum object outside the
    // enumerators' range is undefined, so read its bytes as an int.
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case MTPD_OK: return "MTPD_OK";
        case MTPD_ERR_NULL: return "MTPD_ERR_NULL";
        case MTPD_ERR_SHAPE: return "MTPD_ERR_SHAPE";
        case MTPD_ERR_ALIGN: return "MTPD_ERR_ALIGN";
        case MTPD_ERR_ALIAS: return "MTPD_ERR_ALIAS";
        case MTPD_ERR_WORKSPACE: return "MTPD_ERR_WORKSPACE";
        case MTPD_ERR_HIP: return "MTPD_ERR_HIP";
    }
    return "MTPD_UNKNOWN";
}

const char* mtpd_last_error(void) { return g_err; }

void mtpd_clear_error(void) { g_err[0] = 0; }

int mtpd_abi_version(void) { return 7; }

const char* mtpd_lmhead_plan(int64_t n_rows, int64_t V, int64_t H) {
    thread_local char buf[160];
    buf[0] = 0;
    if (n_rows < 1 || n_rows > kMaxRows || H < mtpd::kBlock || H > kMaxH || H % mtpd::kBlock ||
        V < mtpd::kBlock || V > kMaxV || V % mtpd::kBlock)
        return buf;
    mtpd::describe_lmhead(n_rows, V, H, buf, sizeof buf);
    return buf;
}

const char* mtpd_draft_tail_plan(int64_t M, int64_t V, int64_t H) {
    thread_local char buf[320];
    buf[0] = 0;
    if (M < 1 || M > kMaxRows || H < mtpd::kBlock || H > kMaxH || H % mtpd::kBlock || V < mtpd::kBlock ||
        V > kMaxV || V % mtpd::kBlock)
        return buf;
    if (mtpd::use_draft_tail1(M, H)) {
        snprintf(buf, sizeof buf, "draft_tail1_kernel grid=%lldx256 (%lld tiles)", (long long)mtpd::draft_tail1_grid(V),
                 (long long)(V / 16));
        return buf;
    }
    char lm[160];
    mtpd::describe_lmhead(M, V, H, lm, sizeof lm);
    if (mtpd::plan_override().norm_quant == 1 && H <= 8192)
        snprintf(buf, sizeof buf, "norm_quant_wave_kernel<%lld> grid=%lldx256 + %s", (long long)((H + 511) / 512),
                 (long long)((M + 3) / 4), lm);
    else
        snprintf(buf, sizeof buf, "norm_quant_kernel<%lld> grid=%lldx256 + %s", (long long)((H + 2047) / 2048),
                 (long long)M, lm);
    return buf;
}

size_t mtpd_workspace_bytes(int64_t n_rows) { return n_rows > kMaxRows ? 0 : mtpd::workspace_bytes(n_rows); }

mtpd_status mtpd_norm_quant(const uint16_t* hidden, const uint16_t* residual, const float* norm_weight, float eps,
                            int64_t M, int64_t H, uint16_t* out_hidden, const mtpd_qact* out_act, void* stream) {
    mtpd_status st = check_norm_args(hidden, residual, norm_weight, M, H, out_hidden, out_act);
    if (st != MTPD_OK || M == 0) return st;
    const size_t mh = (size_t)M * (size_t)H;
    const Range outs[] = {{out_hidden, mh * 2, "out_hidden"},
                          {out_act->codes, mh, "out_act.codes"},
                          {out_act->scales, mh / 128 * 4, "out_act.scales"}};
    const Range ins[] = {{hidden, mh * 2, "hidden"}, {residual, mh * 2, "residual"}, {norm_weight, (size_t)H * 4, "norm_weight"}};
    st = check_alias(outs, 3, ins, 3);
    if (st != MTPD_OK) return st;
    return hip_status(mtpd::launch_norm_quant(hidden, residual, norm_weight, eps, M, H, out_hidden, out_act->codes,
                                              out_act->scales, (hipStream_t)stream),
                      "norm_quant launch");
}

mtpd_status mtpd_fp8_lmhead_argmax(const mtpd_qact* act, const int32_t* row_index, int64_t n_rows,
                                   const mtpd_fp8_weight* w, float* out_max, int32_t* out_idx, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!act) return fail(MTPD_ERR_NULL, "act descriptor is NULL");
    if (n_rows < 0 || n_rows > kMaxRows) return fail(MTPD_ERR_SHAPE, "n_rows=%lld out of [0, 2^24]", (long long)n_rows);
    mtpd_status st = check_H(act->cols);
    if (st != MTPD_OK) return st;
    st = check_weight(w, act->cols);
    if (st != MTPD_OK) return st;
    if (n_rows == 0) return MTPD_OK;
    if (act->rows < 1 || act->rows > kMaxRows)
        return fail(MTPD_ERR_SHAPE, "act rows=%lld out of [1, 2^24]", (long long)act->rows);
    if (!row_index && n_rows > act->rows)
        return fail(MTPD_ERR_SHAPE, "n_rows=%lld exceeds act rows=%lld with no row_index", (long long)n_rows,
                    (long long)act->rows);
    if (!act->codes || !act->scales) return fail(MTPD_ERR_NULL, "act codes/scales pointer is NULL");
    if (!aligned(act->codes, 16)) return fail(MTPD_ERR_ALIGN, "act codes not 16-byte aligned");
    if (!aligned(act->scales, 4)) return fail(MTPD_ERR_ALIGN, "act scales not 4-byte aligned");
    if (row_index && !aligned(row_index, 4)) return fail(MTPD_ERR_ALIGN, "row_index not 4-byte aligned");
    st = check_lmhead_outputs(n_rows, out_max, out_idx, workspace, workspace_bytes);
    if (st != MTPD_OK) return st;
    const size_t ah = (size_t)act->rows * (size_t)act->cols;
    const Range outs[] = {{out_max, (size_t)n_rows * 4, "out_max"},
                          {out_idx, (size_t)n_rows * 4, "out_idx"},
                          {workspace, mtpd::workspace_bytes(n_rows), "workspace"}};
    const Range ins[] = {{act->codes, ah, "act.codes"},
                         {act->scales, ah / 128 * 4, "act.scales"},
                         {row_index, row_index ? (size_t)n_rows * 4 : 0, "row_index"},
                         {w->codes, (size_t)w->V * (size_t)w->H, "w.codes"},
                         {w->scales, (size_t)(w->V / 128) * (size_t)(w->H / 128) * 4, "w.scales"}};
    st = check_alias(outs, 3, ins, 5);
    if (st != MTPD_OK) return st;
    mtpd::LmheadArgs a{act->codes, act->scales, row_index, n_rows, act->rows, w->codes, w->scales, w->V, w->H,
                       out_max, out_idx, workspace};
    return hip_status(mtpd::launch_lmhead_argmax(a, (hipStream_t)stream), "lmhead_argmax launch");
}

static mtpd_status draft_tail_impl(const uint16_t* hidden, const uint16_t* residual, const float* norm_weight, float eps,
                            int64_t M, int64_t H, const mtpd_fp8_weight* w, uint16_t* out_hidden,
                            const mtpd_qact* out_act, float* out_max, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, void* stream) {
    mtpd_status st = check_norm_args(hidden, residual, norm_weight, M, H, out_hidden, out_act);
    if (st != MTPD_OK) return st;
    st = check_weight(w, H);
    if (st != MTPD_OK) return st;
    if (M == 0) return MTPD_OK;
    st = check_lmhead_outputs(M, out_max, out_idx, workspace, workspace_bytes);
    if (st != MTPD_OK) return st;
    const size_t mh = (size_t)M * (size_t)H;
    const Range outs[] = {{out_hidden, mh * 2, "out_hidden"},
                          {out_act->codes, mh, "out_act.codes"},
                          {out_act->scales, mh / 128 * 4, "out_act.scales"},
                          {out_max, (size_t)M * 4, "out_max"},
                          {out_idx, (size_t)M * 4, "out_idx"},
                          {workspace, mtpd::workspace_bytes(M), "workspace"}};
    const Range ins[] = {{hidden, mh * 2, "hidden"},
                         {residual, mh * 2, "residual"},
                         {norm_weight, (size_t)H * 4, "norm_weight"},
                         {w->codes, (size_t)w->V * (size_t)H, "w.codes"},
                         {w->scales, (size_t)(w->V / 128) * (size_t)(H / 128) * 4, "w.scales"}};
    st = check_alias(outs, 6, ins, 5);
    if (st != MTPD_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    if (mtpd::use_draft_tail1(M, H))
        return hip_status(mtpd::launch_draft_tail1(hidden, residual, norm_weight, eps, H, w->codes, w->scales, w->V,
                                                   out_hidden, out_act->codes, out_act->scales, out_max, out_idx,
                                                   workspace, s),
                          "draft_tail launch");
    st = hip_status(mtpd::launch_norm_quant(hidden, residual, norm_weight, eps, M, H, out_hidden, out_act->codes,
                                            out_act->scales, s),
                    "norm_quant launch");
    if (st != MTPD_OK) return st;
    mtpd::LmheadArgs a{out_act->codes, out_act->scales, nullptr, M, M, w->codes, w->scales, w->V, H,
                       out_max, out_idx, workspace};
    return hip_status(mtpd::launch_lmhead_argmax(a, s), "lmhead_argmax launch");
}

mtpd_status mtpd_draft_tail(const uint16_t* hidden, const uint16_t* residual, const float* norm_weight, float eps,
                            int64_t M, int64_t H, const mtpd_fp8_weight* w, uint16_t* out_hidden,
                            const mtpd_qact* out_act, float* out_max, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return draft_tail_impl(hidden, residual, norm_weight, eps, M, H, w, out_hidden, out_act, out_max, out_idx,
                           workspace, workspace_bytes, stream);
}

mtpd_status mtpd_draft_tail_noalloc(const uint16_t* hidden, const uint16_t* residual, const float* norm_weight,
                                    float eps, int64_t M, int64_t H, const mtpd_fp8_weight* w, uint16_t* out_hidden,
                                    const mtpd_qact* out_act, float* out_max, int32_t* out_idx, void* stream) {
    if (M > kNoallocMaxRows)
        return fail(MTPD_ERR_WORKSPACE, "M=%lld exceeds the %lld rows the no-alloc scratch holds", (long long)M,
                    (long long)kNoallocMaxRows);
    if (M <= 0) {   // argument checks only; nothing is launched
        return draft_tail_impl(hidden, residual, norm_weight, eps, M, H, w, out_hidden, out_act, out_max, out_idx,
                               nullptr, 0, stream);
    }
    int dev = -1;
    mtpd_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
    if (st != MTPD_OK) return st;
    if (dev < 0 || dev >= kMaxDevices) return fail(MTPD_ERR_HIP, "device %d out of range", dev);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (st != MTPD_OK) return st;
        g_scratch_ptr[dev] = ptr;
    }
    void* ptr = g_scratch_ptr[dev];
    if (!g_scratch_zeroed[dev]) {
        // the keys and counters must start at zero; every completed call
        // leaves them zero again.  A fill kernel, not a memset, so that a
        // first call inside a graph capture stays correct on every replay.
        hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, (uint4*)ptr,
                           kScratchBytes / 16);
        st = hip_status(hipGetLastError(), "scratch zero-fill launch");
        if (st != MTPD_OK) return st;
        g_scratch_zeroed[dev] = true;
    }
    return draft_tail_impl(hidden, residual, norm_weight, eps, M, H, w, out_hidden, out_act, out_max, out_idx, ptr,
                           kScratchBytes, stream);
}

mtpd_status mtpd_allreduce_norm_quant(const uint16_t* const* partials, int64_t n_partials, const uint16_t* residual,
                                      const float* norm_weight, float eps, int64_t M, int64_t H, uint16_t* out_hidden,
                                      const mtpd_qact* out_act, void* stream) {
    if (n_partials < 1 || n_partials > mtpd::kMaxPartials)
        return fail(MTPD_ERR_SHAPE, "n_partials=%lld out of [1, %d]", (long long)n_partials, mtpd::kMaxPartials);
    if (!partials) return fail(MTPD_ERR_NULL, "partials array is NULL");
    mtpd_status st = check_norm_args(partials[0], residual, norm_weight, M, H, out_hidden, out_act);
    if (st != MTPD_OK || M == 0) return st;
    const size_t mh = (size_t)M * (size_t)H;
    mtpd::PartialPtrs parts{};
    parts.n = (int)n_partials;
    Range ins[mtpd::kMaxPartials + 2];
    for (int64_t q = 0; q < n_partials; ++q) {
        if (!partials[q]) return fail(MTPD_ERR_NULL, "partials[%lld] is NULL", (long long)q);
        if (!aligned(partials[q], 16)) return fail(MTPD_ERR_ALIGN, "partials[%lld] not 16-byte aligned", (long long)q);
        parts.p[q] = partials[q];
        ins[q] = Range{partials[q], mh * 2, "a partial"};
    }
    ins[n_partials] = Range{residual, mh * 2, "residual"};
    ins[n_partials + 1] = Range{norm_weight, (size_t)H * 4, "norm_weight"};
    const Range outs[] = {{out_hidden, mh * 2, "out_hidden"},
                          {out_act->codes, mh, "out_act.codes"},
                          {out_act->scales, mh / 128 * 4, "out_act.scales"}};
    st = check_alias(outs, 3, ins, (int)n_partials + 2);
    if (st != MTPD_OK) return st;
    return hip_status(mtpd::launch_allreduce_norm_quant(parts, residual, norm_weight, eps, M, H, out_hidden,
                                                        out_act->codes, out_act->scales, (hipStream_t)stream),
                      "allreduce_norm_quant launch");
}

mtpd_status mtpd_argmax_combine(const float* local_max, const int32_t* local_idx, const int64_t* shard_offset,
                                int64_t n_shards, int64_t n_rows, float* out_max, int32_t* out_idx, void* stream) {
    if (n_shards < 1 || n_shards > mtpd::kMaxShards)
        return fail(MTPD_ERR_SHAPE, "n_shards=%lld out of [1, %d]", (long long)n_shards, mtpd::kMaxShards);
    if (n_rows < 0 || n_rows > kMaxRows) return fail(MTPD_ERR_SHAPE, "n_rows=%lld out of [0, 2^24]", (long long)n_rows);
    if (!shard_offset) return fail(MTPD_ERR_NULL, "shard_offset is NULL");
    mtpd::ShardOffsets offs{};
    for (int64_t s = 0; s < n_shards; ++s) {
        if (shard_offset[s] < 0 || shard_offset[s] > kMaxV)
            return fail(MTPD_ERR_SHAPE, "shard_offset[%lld]=%lld out of [0, 2^31-128]", (long long)s,
                        (long long)shard_offset[s]);
        offs.off[s] = (uint32_t)shard_offset[s];
    }
    if (n_rows == 0) return MTPD_OK;
    if (!local_max || !local_idx || !out_max || !out_idx) return fail(MTPD_ERR_NULL, "a required pointer is NULL");
    if (!aligned(local_max, 4) || !aligned(local_idx, 4) || !aligned(out_max, 4) || !aligned(out_idx, 4))
        return fail(MTPD_ERR_ALIGN, "max/index arrays must be 4-byte aligned");
    const size_t pairs = (size_t)n_shards * (size_t)n_rows;
    const Range outs[] = {{out_max, (size_t)n_rows * 4, "out_max"}, {out_idx, (size_t)n_rows * 4, "out_idx"}};
    const Range ins[] = {{local_max, pairs * 4, "local_max"}, {local_idx, pairs * 4, "local_idx"}};
    mtpd_status st = check_alias(outs, 2, ins, 2);
    if (st != MTPD_OK) return st;
    return hip_status(mtpd::launch_argmax_combine(local_max, local_idx, offs, (int)n_shards, n_rows, out_max, out_idx,
                                                  (hipStream_t)stream),
                      "argmax_combine launch");
}

mtpd_status mtpd_topk_combine(const float* local_val, const int32_t* local_idx, const int64_t* shard_offset,
                              int64_t n_shards, int64_t n_rows, int64_t k, float* out_val, int32_t* out_idx,
                              void* stream) {
    if (n_shards < 1 || n_shards > mtpd::kMaxShards)
        return fail(MTPD_ERR_SHAPE, "n_shards=%lld out of [1, %d]", (long long)n_shards, mtpd::kMaxShards);
    if (n_rows < 0 || n_rows > kMaxRows) return fail(MTPD_ERR_SHAPE, "n_rows=%lld out of [0, 2^24]", (long long)n_rows);
    if (k < 1 || k > mtpd::kMaxTopk) return fail(MTPD_ERR_SHAPE, "k=%lld out of [1, %d]", (long long)k, mtpd::kMaxTopk);
    if (!shard_offset) return fail(MTPD_ERR_NULL, "shard_offset is NULL");
    mtpd::ShardOffsets offs{};
    for (int64_t s = 0; s < n_shards; ++s) {
        if (shard_offset[s] < 0 || shard_offset[s] > kMaxV)
            return fail(MTPD_ERR_SHAPE, "shard_offset[%lld]=%lld out of [0, 2^31-128]", (long long)s,
                        (long long)shard_offset[s]);
        offs.off[s] = (uint32_t)shard_offset[s];
    }
    if (n_rows == 0) return MTPD_OK;
    if (!local_val || !local_idx || !out_val || !out_idx) return fail(MTPD_ERR_NULL, "a required pointer is NULL");
    if (!aligned(local_val, 4) || !aligned(local_idx, 4) || !aligned(out_val, 4) || !aligned(out_idx, 4))
        return fail(MTPD_ERR_ALIGN, "value/index arrays must be 4-byte aligned");
    const size_t cand = (size_t)n_shards * (size_t)n_rows * (size_t)k, outn = (size_t)n_rows * (size_t)k;
    const Range outs[] = {{out_val, outn * 4, "out_val"}, {out_idx, outn * 4, "out_idx"}};
    const Range ins[] = {{local_val, cand * 4, "local_val"}, {local_idx, cand * 4, "local_idx"}};
    mtpd_status st = check_alias(outs, 2, ins, 2);
    if (st != MTPD_OK) return st;
    return hip_status(mtpd::launch_topk_combine(local_val, local_idx, offs, (int)n_shards, n_rows, (int)k, out_val,
                                                out_idx, (hipStream_t)stream),
                      "topk_combine launch");
}

size_t mtpd_topk_workspace_bytes(int64_t n_rows, int64_t V, int64_t k) {
    if (n_rows <= 0 || n_rows > kMaxRows || k < 1 || k > 32 || V < mtpd::kBlock || V > kMaxV || V % mtpd::kBlock)
        return 0;
    return mtpd::topk_workspace_bytes(n_rows, V, k);
}

mtpd_status mtpd_fp8_lmhead_topk(const mtpd_qact* act, const int32_t* row_index, int64_t n_rows,
                                 const mtpd_fp8_weight* w, int64_t k, float* out_val, int32_t* out_idx,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (!act) return fail(MTPD_ERR_NULL, "act descriptor is NULL");
    if (n_rows < 0 || n_rows > kMaxRows) return fail(MTPD_ERR_SHAPE, "n_rows=%lld out of [0, 2^24]", (long long)n_rows);
    if (k < 1 || k > 32) return fail(MTPD_ERR_SHAPE, "k=%lld out of [1, 32]", (long long)k);
    mtpd_status st = check_H(act->cols);
    if (st != MTPD_OK) return st;
    st = check_weight(w, act->cols);
    if (st != MTPD_OK) return st;
    if (n_rows == 0) return MTPD_OK;
    if (act->rows < 1 || act->rows > kMaxRows)
        return fail(MTPD_ERR_SHAPE, "act rows=%lld out of [1, 2^24]", (long long)act->rows);
    if (!row_index && n_rows > act->rows)
        return fail(MTPD_ERR_SHAPE, "n_rows=%lld exceeds act rows=%lld with no row_index", (long long)n_rows,
                    (long long)act->rows);
    if (!mtpd::topk_supported(act->cols, act->rows))
        return fail(MTPD_ERR_SHAPE, "top-k takes H <= 8192 and act rows * H <= 2^32 (H=%lld, rows=%lld)",
                    (long long)act->cols, (long long)act->rows);
    if (!act->codes || !act->scales) return fail(MTPD_ERR_NULL, "act codes/scales pointer is NULL");
    if (!out_val || !out_idx) return fail(MTPD_ERR_NULL, "out_val/out_idx is NULL");
    if (!aligned(act->codes, 16)) return fail(MTPD_ERR_ALIGN, "act codes not 16-byte aligned");
    if (!aligned(act->scales, 4)) return fail(MTPD_ERR_ALIGN, "act scales not 4-byte aligned");
    if (row_index && !aligned(row_index, 4)) return fail(MTPD_ERR_ALIGN, "row_index not 4-byte aligned");
    if (!aligned(out_val, 4) || !aligned(out_idx, 4)) return fail(MTPD_ERR_ALIGN, "out_val/out_idx not 4-byte aligned");
    const size_t need = mtpd::topk_workspace_bytes(n_rows, w->V, k);
    if (!workspace || workspace_bytes < need)
        return fail(MTPD_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", workspace_bytes, workspace,
                    need);
    if (!aligned(workspace, 256)) return fail(MTPD_ERR_ALIGN, "workspace not 256-byte aligned");
    const size_t ah = (size_t)act->rows * (size_t)act->cols;
    const size_t nk = (size_t)n_rows * (size_t)k;
    const Range outs[] = {{out_val, nk * 4, "out_val"}, {out_idx, nk * 4, "out_idx"}, {workspace, need, "workspace"}};
    const Range ins[] = {{act->codes, ah, "act.codes"},
                         {act->scales, ah / 128 * 4, "act.scales"},
                         {row_index, row_index ? (size_t)n_rows * 4 : 0, "row_index"},
                         {w->codes, (size_t)w->V * (size_t)w->H, "w.codes"},
                         {w->scales, (size_t)(w->V / 128) * (size_t)(w->H / 128) * 4, "w.scales"}};
    st = check_alias(outs, 3, ins, 5);
    if (st != MTPD_OK) return st;
    const int64_t KB = act->cols / 128;
    const int cus = mtpd::device_cus();
    for (int64_t c = 0; c < n_rows; c += 64) {
        const int64_t n = n_rows - c < 64 ? n_rows - c : 64;
        mtpd::LmheadArgs a{act->codes, act->scales, row_index ? row_index + c : nullptr, n, act->rows,
                           w->codes, w->scales, w->V, w->H, nullptr, nullptr, workspace};
        if (!row_index) {   // rows c .. c + n - 1 of the activation
            a.a_codes = act->codes + (size_t)c * (size_t)act->cols;
            a.a_scales = act->scales + (size_t)c * (size_t)KB;
            a.a_rows = act->rows - c;
        }
        st = hip_status(mtpd::launch_lmhead_topk(a, (int)k, out_val + (size_t)c * (size_t)k,
                                                 out_idx + (size_t)c * (size_t)k, cus, (hipStream_t)stream),
                        "lmhead_topk launch");
        if (st != MTPD_OK) return st;
    }
    return MTPD_OK;
}

}  // extern "C"
