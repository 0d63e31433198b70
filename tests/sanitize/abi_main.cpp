// Host AddressSanitizer / UndefinedBehaviorSanitizer driver of libmtpd's
// host code (argument validation, size arithmetic, plan strings, the plan
// override parser, the error slot).  Built host-only (no device code) by
// tests/test_sanitizers.py from the library's own sources.  The pointers
// passed are never dereferenced by the validation; every call here fails
// validation or is empty (M == 0), so no HIP call is reached, except the
// few that ask the runtime for a device and get an error without a GPU.
// Prints "abi sanitizer run ok" and exits 0 when nothing fired.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mtpd.h"

#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                         \
        }                                                                     \
    } while (0)

namespace {

alignas(256) unsigned char arena[1 << 16];
template <class T> T* at(size_t off) { return reinterpret_cast<T*>(arena + off); }

}  // namespace

int main() {
    const int64_t big[] = {-1, 0, 1, 63, 64, 65, 4096, 65536, 1 << 24, (1 << 24) + 1, INT64_C(1) << 40,
                           INT64_MAX};
    for (int s = -1; s < 9; ++s) CHECK(mtpd_status_name((mtpd_status)s) != nullptr);
    for (int64_t n : big) {
        (void)mtpd_workspace_bytes(n);
        for (int64_t v : big)
            for (int64_t k : {INT64_C(-1), INT64_C(0), INT64_C(1), INT64_C(32), INT64_C(33), INT64_MAX})
                (void)mtpd_topk_workspace_bytes(n, v, k);
        for (int64_t v : big)
            for (int64_t h : {INT64_C(0), INT64_C(128), INT64_C(6144), INT64_C(16384), INT64_MAX}) {
                CHECK(mtpd_lmhead_plan(n, v, h) != nullptr);
                CHECK(mtpd_draft_tail_plan(n, v, h) != nullptr);
            }
    }

    // plan override parser: valid, invalid, long and empty strings
    char longv[4096];
    std::memset(longv, '7', sizeof longv - 1);
    longv[sizeof longv - 1] = 0;
    const char* keys[] = {"lmhead_kernel", "lmhead_tile", "lmhead_stream", "lmhead_rows", "lmhead_decode",
                          "lmhead_kouter", "lmhead_gemm", "draft_tail", "device_cus", "bogus", ""};
    const char* vals[] = {"generic", "decode", "1,2,3", "4,2", "0", "1,2,3,4", "-1", "1,,2", ",", "99999999999999",
                          "split", "", "a", longv, nullptr};
    for (const char* k : keys)
        for (const char* v : vals) (void)mtpd_set_plan_override(k, v);
    CHECK(mtpd_set_plan_override(nullptr, nullptr) == MTPD_OK);
    CHECK(mtpd_set_plan_override("bogus", "1") == MTPD_ERR_SHAPE);

    uint16_t* hid = at<uint16_t>(0);
    uint16_t* res = at<uint16_t>(8192);
    float* g = at<float>(16384);
    uint16_t* oh = at<uint16_t>(20480);
    mtpd_qact qa{at<uint8_t>(28672), at<float>(32768), 4, 256};
    mtpd_qact qa0{at<uint8_t>(28672), at<float>(32768), 0, 256};   // for the empty (M == 0) calls
    mtpd_fp8_weight w{at<uint8_t>(36864), at<float>(45056), 256, 256};
    float* omax = at<float>(49152);
    int32_t* oidx = at<int32_t>(49664);
    void* wsp = at<void>(53248);
    const int64_t M = 4, H = 256;

    // empty calls and every validation failure class
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, 0, H, oh, &qa0, nullptr) == MTPD_OK);
    CHECK(mtpd_norm_quant(nullptr, res, g, 1e-6f, M, H, oh, &qa, nullptr) == MTPD_ERR_NULL);
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, M, 100, oh, &qa, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, -1, H, oh, &qa, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, INT64_C(1) << 40, INT64_C(1) << 40, oh, &qa, nullptr) ==
          MTPD_ERR_SHAPE);
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, INT64_MAX, H, oh, &qa, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_norm_quant(at<uint16_t>(2), res, g, 1e-6f, M, H, oh, &qa, nullptr) == MTPD_ERR_ALIGN);
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, M, H, hid, &qa, nullptr) == MTPD_ERR_ALIAS);
    CHECK(mtpd_norm_quant(hid, res, g, 1e-6f, M, H, oh, nullptr, nullptr) == MTPD_ERR_NULL);

    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, 0, &w, omax, oidx, wsp, 4096, nullptr) == MTPD_OK);
    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, M, &w, omax, oidx, nullptr, 0, nullptr) == MTPD_ERR_WORKSPACE);
    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, M, &w, omax, oidx, wsp, 1, nullptr) == MTPD_ERR_WORKSPACE);
    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, M, nullptr, omax, oidx, wsp, 4096, nullptr) == MTPD_ERR_NULL);
    mtpd_fp8_weight wbad = w;
    wbad.V = 200;
    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, M, &wbad, omax, oidx, wsp, 4096, nullptr) == MTPD_ERR_SHAPE);
    wbad.V = INT64_MAX - 127;
    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, M, &wbad, omax, oidx, wsp, 4096, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_fp8_lmhead_argmax(&qa, nullptr, INT64_MAX, &w, omax, oidx, wsp, 4096, nullptr) == MTPD_ERR_SHAPE);

    CHECK(mtpd_draft_tail(hid, res, g, 1e-6f, 0, H, &w, oh, &qa0, omax, oidx, wsp, 4096, nullptr) == MTPD_OK);
    CHECK(mtpd_draft_tail(hid, res, g, 1e-6f, M, H, &w, oh, &qa, omax, oidx, nullptr, 0, nullptr) ==
          MTPD_ERR_WORKSPACE);
    CHECK(mtpd_draft_tail(hid, res, g, 1e-6f, M, H, &w, oh, &qa, at<float>(2), oidx, wsp, 4096, nullptr) ==
          MTPD_ERR_ALIGN);
    CHECK(mtpd_draft_tail_noalloc(hid, res, g, 1e-6f, 65537, H, &w, oh, &qa, omax, oidx, nullptr) ==
          MTPD_ERR_WORKSPACE);
    CHECK(mtpd_draft_tail_noalloc(hid, res, g, 1e-6f, 0, H, &w, oh, &qa0, omax, oidx, nullptr) == MTPD_OK);
    CHECK(mtpd_draft_tail_noalloc(nullptr, res, g, 1e-6f, -5, H, &w, oh, &qa, omax, oidx, nullptr) != MTPD_OK);

    const uint16_t* parts[17] = {hid, res, hid, res, hid, res, hid, res, hid, res, hid, res, hid, res, hid, res, hid};
    CHECK(mtpd_allreduce_norm_quant(parts, 0, res, g, 1e-6f, M, H, oh, &qa, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_allreduce_norm_quant(parts, 17, res, g, 1e-6f, M, H, oh, &qa, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_allreduce_norm_quant(nullptr, 2, res, g, 1e-6f, M, H, oh, &qa, nullptr) == MTPD_ERR_NULL);
    CHECK(mtpd_allreduce_norm_quant(parts, 2, res, g, 1e-6f, 0, H, oh, &qa0, nullptr) == MTPD_OK);

    const int64_t offs[3] = {0, 256, 512};
    CHECK(mtpd_argmax_combine(omax, oidx, offs, 0, M, at<float>(57344), at<int32_t>(57856), nullptr) ==
          MTPD_ERR_SHAPE);
    CHECK(mtpd_argmax_combine(omax, oidx, offs, 65, M, at<float>(57344), at<int32_t>(57856), nullptr) ==
          MTPD_ERR_SHAPE);
    CHECK(mtpd_argmax_combine(omax, oidx, nullptr, 3, M, at<float>(57344), at<int32_t>(57856), nullptr) ==
          MTPD_ERR_NULL);
    CHECK(mtpd_argmax_combine(omax, oidx, offs, 3, 0, at<float>(57344), at<int32_t>(57856), nullptr) == MTPD_OK);

    for (int64_t k : {INT64_C(0), INT64_C(33), INT64_C(-1), INT64_MAX})
        CHECK(mtpd_topk_combine(omax, oidx, offs, 3, M, k, at<float>(57344), at<int32_t>(57856), nullptr) ==
              MTPD_ERR_SHAPE);
    CHECK(mtpd_topk_combine(omax, oidx, offs, 65, M, 8, at<float>(57344), at<int32_t>(57856), nullptr) ==
          MTPD_ERR_SHAPE);
    CHECK(mtpd_topk_combine(omax, oidx, nullptr, 3, M, 8, at<float>(57344), at<int32_t>(57856), nullptr) ==
          MTPD_ERR_NULL);
    CHECK(mtpd_topk_combine(omax, oidx, offs, 3, 0, 8, at<float>(57344), at<int32_t>(57856), nullptr) == MTPD_OK);

    for (int64_t k : {INT64_C(0), INT64_C(33), INT64_C(-1), INT64_MAX})
        CHECK(mtpd_fp8_lmhead_topk(&qa, nullptr, M, &w, k, omax, oidx, wsp, 4096, nullptr) == MTPD_ERR_SHAPE);
    CHECK(mtpd_fp8_lmhead_topk(&qa, nullptr, 0, &w, 8, omax, oidx, wsp, 4096, nullptr) == MTPD_OK);

    // the error slot keeps the first failure until cleared
    mtpd_clear_error();
    CHECK(mtpd_last_error()[0] == 0);
    (void)mtpd_norm_quant(nullptr, res, g, 1e-6f, M, H, oh, &qa, nullptr);
    char first[512];
    std::snprintf(first, sizeof first, "%s", mtpd_last_error());
    (void)mtpd_norm_quant(hid, res, g, 1e-6f, M, 100, oh, &qa, nullptr);
    CHECK(std::strcmp(first, mtpd_last_error()) == 0);
    mtpd_clear_error();
    CHECK(mtpd_abi_version() == 7);
    std::printf("abi sanitizer run ok\n");
    return 0;
}
