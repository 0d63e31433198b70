/*
 * Host AddressSanitizer / UndefinedBehaviorSanitizer driver of the CPU
 * oracle: every exported oracle function on small ragged shapes (several
 * 128-column blocks, vocab not a multiple of the oracle's chunk, a row
 * subset, zero rows and zero-valued blocks), with a few structural checks.
 * Built by tests/test_sanitizers.py with -fsanitize=address,undefined;
 * prints "oracle sanitizer run ok" and exits 0 when nothing fired.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double ora_e4m3_decode(uint8_t c);
uint8_t ora_e4m3_encode(double x);
double ora_bf16_decode(uint16_t b);
uint16_t ora_bf16_encode(double x);
void ora_e4m3_encode_array(const double *x, int64_t n, uint8_t *out);
void ora_bf16_encode_array(const double *x, int64_t n, uint16_t *out);
void ora_block_quant(const double *y, int64_t M, int64_t H, uint8_t *codes, float *scales);
void ora_norm_quant(const uint16_t *hidden, const uint16_t *residual, const float *norm_weight, float eps,
                    int64_t M, int64_t H, uint16_t *out_hidden, uint8_t *codes, float *scales, double *y_out,
                    double *rstd_out);
void ora_allreduce_norm_quant(const uint16_t *partials, int64_t P, const uint16_t *residual,
                              const float *norm_weight, float eps, int64_t M, int64_t H, uint16_t *out_hidden,
                              uint8_t *codes, float *scales, double *y_out, double *rstd_out);
void ora_logits(const uint8_t *act_codes, const float *act_scales, int64_t H, const int32_t *rows,
                int64_t n_rows, const uint8_t *w_codes, const float *w_scales, int64_t V, double *z_out);
void ora_argmax(const uint8_t *act_codes, const float *act_scales, int64_t H, const int32_t *rows,
                int64_t n_rows, const uint8_t *w_codes, const float *w_scales, int64_t V, float *out_max,
                int32_t *out_idx, double *out_z1, double *out_z2);
void ora_topk(const uint8_t *act_codes, const float *act_scales, int64_t H, const int32_t *rows,
              int64_t n_rows, const uint8_t *w_codes, const float *w_scales, int64_t V, int64_t k,
              float *out_val, int32_t *out_idx);
int ora_num_threads(void);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* xorshift64*, in [-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main(void) {
    enum { M = 5, H = 384, KB = H / 128, V = 640, P = 3, K = 7, NR = 3 };
    int i, j;
    CHECK(ora_num_threads() >= 1);
    for (i = 0; i < 256; ++i) {
        const double d = ora_e4m3_decode((uint8_t)i);
        if (!isnan(d)) CHECK(ora_e4m3_decode(ora_e4m3_encode(d)) == d || d == 0.0);
    }
    for (i = 0; i < 65536; i += 7) {
        const double d = ora_bf16_decode((uint16_t)i);
        if (!isnan(d)) CHECK(ora_bf16_decode(ora_bf16_encode(d)) == d || d == 0.0);
    }
    {
        const double x[6] = {0.0, -0.0, 1e300, -1e-300, 448.0, 464.0};
        uint8_t c[6];
        uint16_t b[6];
        ora_e4m3_encode_array(x, 6, c);
        ora_bf16_encode_array(x, 6, b);
        CHECK(c[4] == 0x7E && c[5] == 0x7E);
    }

    uint16_t *hid = malloc(sizeof(uint16_t) * M * H), *res = malloc(sizeof(uint16_t) * M * H);
    uint16_t *parts = malloc(sizeof(uint16_t) * P * M * H), *oh = malloc(sizeof(uint16_t) * M * H);
    float *g = malloc(sizeof(float) * H), *sc = malloc(sizeof(float) * M * KB);
    uint8_t *codes = malloc((size_t)M * H);
    double *y = malloc(sizeof(double) * M * H), *rstd = malloc(sizeof(double) * M);
    uint8_t *wc = malloc((size_t)V * H);
    float *ws = malloc(sizeof(float) * (V / 128) * KB);
    for (i = 0; i < M * H; ++i) {
        hid[i] = ora_bf16_encode(uniform() * 4.0);
        res[i] = ora_bf16_encode(uniform());
    }
    for (i = 0; i < H; ++i) hid[2 * H + i] = res[2 * H + i] = 0;   /* an all-zero row */
    for (i = 0; i < P * M * H; ++i) parts[i] = ora_bf16_encode(uniform());
    for (i = 0; i < H; ++i) g[i] = (float)(1.0 + 0.25 * uniform());
    for (i = 0; i < V * H; ++i) wc[i] = (uint8_t)(((state = state * 6364136223846793005ull + 1) >> 56) & 0xFE) & 0x7E;
    for (i = 0; i < (V / 128) * KB; ++i) ws[i] = (float)(0.01 * (1.5 + uniform()));

    ora_norm_quant(hid, res, g, 1e-6f, M, H, oh, codes, sc, y, rstd);
    for (j = 0; j < KB; ++j) CHECK(sc[2 * KB + j] == 0.0f);
    for (i = 0; i < M * KB; ++i) CHECK(sc[i] >= 0.0f && isfinite(sc[i]));
    ora_norm_quant(hid, res, g, 1e-6f, 0, H, oh, codes, sc, NULL, NULL);
    ora_allreduce_norm_quant(parts, P, res, g, 1e-6f, M, H, oh, codes, sc, y, rstd);
    ora_block_quant(y, M, H, codes, sc);

    double *z = malloc(sizeof(double) * M * V);
    const int32_t rows[NR] = {4, 0, 4};
    ora_logits(codes, sc, H, NULL, M, wc, ws, V, z);
    ora_logits(codes, sc, H, rows, NR, wc, ws, V, z);
    float mx[M], val[M * K];
    int32_t idx[M], tidx[M * K];
    double z1[M], z2[M];
    ora_argmax(codes, sc, H, NULL, M, wc, ws, V, mx, idx, z1, z2);
    for (i = 0; i < M; ++i) CHECK(idx[i] >= 0 && idx[i] < V && z1[i] >= z2[i]);
    ora_argmax(codes, sc, H, rows, NR, wc, ws, V, mx, idx, z1, z2);
    ora_topk(codes, sc, H, rows, NR, wc, ws, V, K, val, tidx);
    for (i = 0; i < NR; ++i)
        for (j = 1; j < K; ++j) CHECK(val[i * K + j - 1] >= val[i * K + j]);
    ora_topk(codes, sc, H, NULL, M, wc, ws, V, 1, val, tidx);

    free(hid); free(res); free(parts); free(oh); free(g); free(sc); free(codes); free(y); free(rstd);
    free(wc); free(ws); free(z);
    printf("oracle sanitizer run ok\n");
    return 0;
}
