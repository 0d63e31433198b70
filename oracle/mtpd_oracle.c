/*
 * CPU oracle for the MTP draft-layer tail.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's
 * cpu_baseline leg load this library.  The product path (the HIP library
 * and its Python binding) never calls it, and this file shares no code,
 * header, table or helper with the HIP sources.
 *
 * What it computes, and where each step is defined:
 *   - residual add, then RMSNorm: the MTP layer's final all-reduce and
 *     RMSNorm ("[Quant][MTP] Reuse packed FP8 logits inputs", Purpose;
 *     "[Spec Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax
 *     draft tokens", Summary).  ora_norm_quant takes the norm input as
 *     hidden + residual (the all-reduce of a single partial is the
 *     identity); ora_allreduce_norm_quant sums P row-parallel partials
 *     first, standing in for the all-reduce on one GPU.
 *   - two outputs of the norm: the bf16 hidden recycled to the next MTP
 *     position and a packed FP8 activation for the shared LM head
 *     ("Reuse packed FP8 logits inputs", Purpose).  Packing is OCP E4M3FN
 *     codes with one fp32 dequant scale per row per 128 columns,
 *     scale = amax/448.
 *   - the LM head consumes the packed activation as it is, never unpacking
 *     and requantizing it ("Reuse packed FP8 logits inputs", Purpose and
 *     Dependencies: block-linear prequantized-input GEMM).  The weight is
 *     E4M3FN codes with one fp32 scale per 128x128 block.
 *   - the greedy draft token is a local argmax over this GPU's vocab slice,
 *     so full-vocab logits are never gathered ("Fuse the MTP trailing
 *     all-reduce; local-argmax draft tokens", Summary and Benchmarks).
 *     Equal maxima resolve to the lowest index.
 *
 * Arithmetic is fp64 throughout, except where the result is defined as an
 * fp32 value: the block scales (an fp32 dequant multiplier) and the logit
 * the argmax is decided on (logits are fp32 and never materialized, so the
 * draft token is the first index of the largest fp32 logit).  The 8-bit
 * code is the E4M3 rounding of the fp64 quotient y / scale, rounded once.
 *
 * Parity pins for every function here live in tests/ (codecs against the
 * library casts of torch, RMSNorm closed forms, quantization invariants,
 * GEMM against a float64 matmul, one-hot closed forms, planted ties).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_BLOCK 128

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN codec, written from the format definition:                  */
/* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinities;     */
/* S.1111.111 is NaN; largest finite magnitude 448 (0x7E); exponent field 0  */
/* holds subnormals m * 2^-9.                                                 */
/* ------------------------------------------------------------------------ */

double ora_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);              /* (m/8) * 2^(1-7) */
    else
        mag = ldexp((double)(8 + m), e - 10);    /* (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/*
 * Round x to the nearest E4M3FN value, ties to the even mantissa, saturating
 * to +-448, keeping the sign (so a small negative value becomes 0x80).
 * Rounding to a floating-point grid: inside the binade [2^E, 2^(E+1)) the
 * representable values are spaced 2^(E-3); below 2^-6 (the smallest normal)
 * the spacing is the subnormal step 2^-9.  a / spacing is exact in fp64
 * (division by a power of two) and nearbyint() rounds half to even in the
 * default rounding mode.  NaN input gives the NaN code 0x7F.
 */
uint8_t ora_e4m3_encode(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    double spacing, r;
    int E;

    if (isnan(x))
        return 0x7F;
    if (a < ldexp(1.0, -6)) {
        spacing = ldexp(1.0, -9);
    } else {
        (void)frexp(a, &E);                       /* a = f * 2^E, f in [0.5, 1) */
        spacing = ldexp(1.0, (E - 1) - 3);
    }
    r = nearbyint(a / spacing) * spacing;
    if (r > 448.0)
        r = 448.0;

    /* encode the finite magnitude r */
    if (r < ldexp(1.0, -6)) {
        /* subnormal (or zero): code = r / 2^-9 in 0..7; r == 2^-6 cannot occur here */
        return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    }
    (void)frexp(r, &E);                           /* r = f * 2^E */
    {
        int ebias = (E - 1) + 7;                  /* biased exponent, 1..15 */
        int mant = (int)(r / ldexp(1.0, E - 1) * 8.0) - 8;   /* 0..7 */
        return (uint8_t)(sign | (uint8_t)(ebias << 3) | (uint8_t)mant);
    }
}

/* ------------------------------------------------------------------------ */
/* bfloat16 codec: the upper half of an IEEE binary32; 8 significant bits.   */
/* ------------------------------------------------------------------------ */

double ora_bf16_decode(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round x to the nearest bfloat16, ties to even.  Normal range: 8
 * significant bits, so inside [2^E, 2^(E+1)) the spacing is 2^(E-7);
 * below 2^-126 the spacing is the subnormal step 2^-133.  The rounded value
 * is representable in binary32, so the final conversion to float is exact;
 * values at or past the overflow threshold become infinity, as in IEEE.
 */
uint16_t ora_bf16_encode(double x)
{
    double a = fabs(x), spacing, r;
    float f;
    uint32_t u;
    int E;

    if (isnan(x))
        return 0x7FC0;
    if (a < ldexp(1.0, -126)) {
        spacing = ldexp(1.0, -133);
    } else {
        (void)frexp(a, &E);
        spacing = ldexp(1.0, (E - 1) - 7);
    }
    r = nearbyint(a / spacing) * spacing;
    if (r >= ldexp(1.0, 128))
        r = INFINITY;
    f = (float)(signbit(x) ? -r : r);
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Array forms of the codecs, for exhaustive and sampled tests. */
void ora_e4m3_encode_array(const double *x, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = ora_e4m3_encode(x[i]);
}

void ora_bf16_encode_array(const double *x, int64_t n, uint16_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = ora_bf16_encode(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Packed FP8 activation: one fp32 scale per row per 128-column block.        */
/* ------------------------------------------------------------------------ */

/*
 * Quantize one row y[0..H) (H a multiple of 128):
 *   amax  = max |y_j| over the block
 *   scale = RN_f32(amax / 448), the dequant multiplier (y ~ dec(code) * scale)
 *   code  = E4M3(y_j / scale), the fp64 quotient rounded once to the
 *           nearest E4M3FN value, ties to even, saturating at +-448
 * A block whose scale is zero (amax zero, or so small the quotient underflows
 * fp32) gets scale 0 and all-zero codes.
 */
static void ora_block_quant_row(const double *y, int64_t H, uint8_t *codes, float *scales)
{
    int64_t b, j, KB = H / ORA_BLOCK;
    for (b = 0; b < KB; ++b) {
        double amax = 0.0;
        float scale;
        for (j = b * ORA_BLOCK; j < (b + 1) * ORA_BLOCK; ++j)
            if (fabs(y[j]) > amax)
                amax = fabs(y[j]);
        scale = (float)(amax / 448.0);
        scales[b] = scale;
        for (j = b * ORA_BLOCK; j < (b + 1) * ORA_BLOCK; ++j) {
            if (scale == 0.0f) {
                codes[j] = 0x00;
            } else {
                codes[j] = ora_e4m3_encode(y[j] / (double)scale);
            }
        }
    }
}

/* y: [M][H] fp64 -> codes [M][H], scales [M][H/128] */
void ora_block_quant(const double *y, int64_t M, int64_t H, uint8_t *codes, float *scales)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m)
        ora_block_quant_row(y + m * H, H, codes + m * H, scales + m * (H / ORA_BLOCK));
}

/* ------------------------------------------------------------------------ */
/* Residual add + RMSNorm + the two outputs.                                  */
/* ------------------------------------------------------------------------ */

/*
 * The norm and the two outputs for one row, from its norm input s[0..H) in
 * fp64 (overwritten with y).  Returns rstd.
 */
static double ora_norm_row(double *s, const float *norm_weight, float eps, int64_t H,
                           uint16_t *out_hidden, uint8_t *codes, float *scales, double *y_out)
{
    double ms = 0.0, rstd;
    int64_t j;

    for (j = 0; j < H; ++j)
        ms += s[j] * s[j];
    ms = ms / (double)H;
    rstd = 1.0 / sqrt(ms + (double)eps);

    for (j = 0; j < H; ++j) {
        s[j] = s[j] * rstd * (double)norm_weight[j];
        out_hidden[j] = ora_bf16_encode(s[j]);
        if (y_out)
            y_out[j] = s[j];
    }
    ora_block_quant_row(s, H, codes, scales);
    return rstd;
}

/*
 * hidden, residual: [M][H] bfloat16 bit patterns, row-major.
 * norm_weight: [H] fp32.  eps: fp32, added to the mean square.
 * Outputs:
 *   out_hidden [M][H] bf16 : RNE_bf16(y), the recycled hidden
 *   codes      [M][H] u8   : packed activation codes (ora_block_quant_row)
 *   scales     [M][H/128]  : its fp32 dequant multipliers
 *   y_out      [M][H] f64  : the unrounded normalized value (may be NULL)
 *   rstd_out   [M] f64     : 1/sqrt(mean(s^2) + eps) (may be NULL)
 *
 * s = hidden + residual is exact in fp64 whenever the two exponents differ
 * by less than 45 (true of every finite input of interest here).
 * y = s * rstd * g.  The norm has no (1 + g) offset; eps sits inside the
 * square root.  Both outputs come from the same unrounded y: the packed
 * activation is not re-derived from the rounded bf16 output.
 */
void ora_norm_quant(const uint16_t *hidden, const uint16_t *residual,
                    const float *norm_weight, float eps, int64_t M, int64_t H,
                    uint16_t *out_hidden, uint8_t *codes, float *scales,
                    double *y_out, double *rstd_out)
{
    int64_t KB = H / ORA_BLOCK;
    int64_t m;

#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        double *s = (double *)malloc((size_t)H * sizeof(double));
        double rstd;
        int64_t j;

        for (j = 0; j < H; ++j)
            s[j] = ora_bf16_decode(hidden[m * H + j]) + ora_bf16_decode(residual[m * H + j]);
        rstd = ora_norm_row(s, norm_weight, eps, H, out_hidden + m * H, codes + m * H, scales + m * KB,
                            y_out ? y_out + m * H : NULL);
        if (rstd_out)
            rstd_out[m] = rstd;
        free(s);
    }
}

/*
 * The same step with the MTP layer's trailing all-reduce in front of the
 * norm ("[Spec Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax
 * draft tokens", Summary): the norm input is the sum of the P row-parallel
 * partial outputs plus the residual,
 *   s = sum_p partials[p] + residual
 * taken in fp64 (exact for bf16 inputs whose exponents span less than about
 * 40 binades), then normalized and packed exactly as ora_norm_quant does.
 * partials: [P][M][H] bf16, contiguous.
 */
void ora_allreduce_norm_quant(const uint16_t *partials, int64_t P, const uint16_t *residual,
                              const float *norm_weight, float eps, int64_t M, int64_t H,
                              uint16_t *out_hidden, uint8_t *codes, float *scales,
                              double *y_out, double *rstd_out)
{
    int64_t KB = H / ORA_BLOCK;
    int64_t m;

#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        double *s = (double *)malloc((size_t)H * sizeof(double));
        double rstd;
        int64_t j, p;

        for (j = 0; j < H; ++j) {
            double acc = 0.0;
            for (p = 0; p < P; ++p)
                acc += ora_bf16_decode(partials[(p * M + m) * H + j]);
            s[j] = acc + ora_bf16_decode(residual[m * H + j]);
        }
        rstd = ora_norm_row(s, norm_weight, eps, H, out_hidden + m * H, codes + m * H, scales + m * KB,
                            y_out ? y_out + m * H : NULL);
        if (rstd_out)
            rstd_out[m] = rstd;
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* Block-scaled FP8 LM head and greedy argmax.                                */
/* ------------------------------------------------------------------------ */

/*
 * z[i][v] = sum_b sa[row_i][b] * sw[v/128][b] * sum_{k in block b} dec(qa[row_i][k]) * dec(qw[v][k])
 *
 * act_codes [A][H] u8, act_scales [A][H/128] f32; rows [n_rows] picks which
 * activation rows (NULL = 0..n_rows-1); w_codes [V][H] u8 (K contiguous),
 * w_scales [V/128][H/128] f32.  z_out: [n_rows][V] fp64.
 * Each inner block sum is exact in fp64 (128 products of two 4-bit
 * significands), so z is the dot product of the dequantized vectors up to
 * the rounding of the block-sum loop.
 */
void ora_logits(const uint8_t *act_codes, const float *act_scales, int64_t H,
                const int32_t *rows, int64_t n_rows,
                const uint8_t *w_codes, const float *w_scales, int64_t V,
                double *z_out)
{
    int64_t KB = H / ORA_BLOCK;
    int64_t VCH = 256;                 /* vocab rows per parallel work item */
    int64_t nch = (V + VCH - 1) / VCH;
    int64_t item;
    double dec[256];
    int c;

    for (c = 0; c < 256; ++c)
        dec[c] = ora_e4m3_decode((uint8_t)c);

#pragma omp parallel for schedule(dynamic, 1)
    for (item = 0; item < n_rows * nch; ++item) {
        int64_t i = item / nch, ch = item % nch;
        int64_t row = rows ? (int64_t)rows[i] : i;
        const uint8_t *qa = act_codes + row * H;
        const float *sa = act_scales + row * KB;
        int64_t v, vend = (ch + 1) * VCH < V ? (ch + 1) * VCH : V;

        for (v = ch * VCH; v < vend; ++v) {
            const uint8_t *qw = w_codes + v * H;
            const float *sw = w_scales + (v / ORA_BLOCK) * KB;
            double z = 0.0;
            int64_t b, k;
            for (b = 0; b < KB; ++b) {
                double inner = 0.0;
                for (k = b * ORA_BLOCK; k < (b + 1) * ORA_BLOCK; ++k)
                    inner += dec[qa[k]] * dec[qw[k]];
                z += (double)sa[b] * (double)sw[b] * inner;
            }
            z_out[i * V + v] = z;
        }
    }
}

/*
 * Greedy local argmax over the V vocab rows of this weight (a whole vocab or
 * one shard of it).  The decision is taken on the fp32 logit: idx is the
 * lowest v whose RN_f32(z[v]) equals the largest RN_f32(z); +0 and -0 are
 * equal.  Returned per row:
 *   out_max  : RN_f32(z[idx])
 *   out_idx  : idx, local to this weight, in [0, V)
 *   out_z1   : z[idx] in fp64
 *   out_z2   : the largest z[v] over v != idx in fp64 (-inf if V == 1),
 *              which the near-tie rule of the tests measures the gap with.
 */
void ora_argmax(const uint8_t *act_codes, const float *act_scales, int64_t H,
                const int32_t *rows, int64_t n_rows,
                const uint8_t *w_codes, const float *w_scales, int64_t V,
                float *out_max, int32_t *out_idx, double *out_z1, double *out_z2)
{
    double *z = (double *)malloc((size_t)(n_rows * V) * sizeof(double));
    int64_t i;

    ora_logits(act_codes, act_scales, H, rows, n_rows, w_codes, w_scales, V, z);

#pragma omp parallel for schedule(static)
    for (i = 0; i < n_rows; ++i) {
        const double *zr = z + i * V;
        int64_t v, best = 0;
        float bestf = (float)zr[0];
        double second = -INFINITY;
        for (v = 1; v < V; ++v) {
            float f = (float)zr[v];
            if (f > bestf) {
                bestf = f;
                best = v;
            }
        }
        for (v = 0; v < V; ++v)
            if (v != best && zr[v] > second)
                second = zr[v];
        out_max[i] = bestf;
        out_idx[i] = (int32_t)best;
        out_z1[i] = zr[best];
        out_z2[i] = second;
    }
    free(z);
}

/*
 * Greedy local top-k: the k vocab rows with the largest fp32 logits, in
 * descending order of the fp32 logit, equal logits in ascending index order
 * (+0 and -0 equal), the same decision rule as ora_argmax (k == 1 gives its
 * result).  The pages compare draft and reference distributions by their
 * top-8 and top-32 sets ("feat(glm52): add checkpoint-native MTP speculative
 * decoding", Accuracy).  out_val, out_idx: [n_rows][k]; 1 <= k <= V.
 * A plain selection: k passes over the row, each taking the best entry not
 * yet taken.
 */
void ora_topk(const uint8_t *act_codes, const float *act_scales, int64_t H,
              const int32_t *rows, int64_t n_rows,
              const uint8_t *w_codes, const float *w_scales, int64_t V, int64_t k,
              float *out_val, int32_t *out_idx)
{
    double *z = (double *)malloc((size_t)(n_rows * V) * sizeof(double));
    int64_t i;

    ora_logits(act_codes, act_scales, H, rows, n_rows, w_codes, w_scales, V, z);

#pragma omp parallel for schedule(static)
    for (i = 0; i < n_rows; ++i) {
        const double *zr = z + i * V;
        unsigned char *taken = (unsigned char *)calloc((size_t)V, 1);
        int64_t e, v;
        for (e = 0; e < k; ++e) {
            int64_t best = -1;
            float bestf = 0.0f;
            for (v = 0; v < V; ++v) {
                float f = (float)zr[v];
                if (taken[v])
                    continue;
                if (best < 0 || f > bestf) {   /* strict: the lowest index wins equal values */
                    best = v;
                    bestf = f;
                }
            }
            taken[best] = 1;
            out_val[i * k + e] = bestf;
            out_idx[i * k + e] = (int32_t)best;
        }
        free(taken);
    }
    free(z);
}

int ora_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
