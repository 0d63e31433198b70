/*
 * mtpd.h -- C ABI of libmtpd, the MTP draft-layer tail on one AMD MI355X
 * (gfx950): residual add + RMSNorm producing a bf16 recycled hidden and a
 * packed FP8 activation, a block-scaled FP8 LM head over that activation,
 * and a fused greedy argmax that never writes logits to memory.
 *
 * Where the operations are defined:
 *   - "[Quant][MTP] Reuse packed FP8 logits inputs", Purpose: the MTP layer
 *     fuses its final all-reduce and RMSNorm with packed FP8 quantization for
 *     the shared LM head and returns two different values, the packed
 *     activation for the logits and the post-norm bf16 hidden for the next
 *     MTP position; consumers index that packed activation and never unpack
 *     and requantize it.  Dependencies: the LM-head GEMM takes the activation
 *     prequantized, block-linear.
 *   - "[Spec Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax
 *     draft tokens", Summary: greedy draft tokens come from a local argmax
 *     over this GPU's vocab slice instead of gathering full-vocab logits.
 *     Accuracy: the fused norm accumulates in fp32.
 *
 * Formats (all row-major, all device memory unless stated):
 *   bf16         uint16 bit patterns of bfloat16.
 *   E4M3 codes   OCP FP8 E4M3FN (max 448, no infinities, 0x7F/0xFF NaN).
 *   packed act   codes [rows][cols] u8 and scales [rows][cols/128] f32; the
 *                value of element (r, c) is dec(code) * scale[r][c/128].
 *   FP8 weight   codes [V][H] u8 (K contiguous) and scales [V/128][H/128]
 *                f32, one per 128x128 block.
 *
 * Conventions shared by every entry point:
 *   - The caller owns all memory; the library allocates nothing and keeps no
 *     state between calls, except the device scratch array of
 *     mtpd_draft_tail_noalloc (and the process-wide plan override).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     null stream) and never synchronizes.
 *   - Arguments are validated on the host before any HIP call; on failure
 *     nothing is launched and a status other than MTPD_OK is returned.  A
 *     failed launch returns MTPD_ERR_HIP.  Faults inside a kernel surface at
 *     the caller's next synchronization.
 *   - The first failure on a thread is kept (mtpd_last_error) until
 *     mtpd_clear_error is called; later failures do not overwrite it.
 *   - Inputs are never written.  Outputs must not overlap inputs or each
 *     other.  Every output element is overwritten.
 *   - Limits: 128 <= H <= 16384 and H % 128 == 0; V % 128 == 0 and
 *     128 <= V <= 2^31 - 128; 0 <= M, n_rows <= 2^24.  M == 0 (or
 *     n_rows == 0) is a valid empty call that launches nothing.
 *   - Alignment: bf16 arrays, code arrays and norm_weight 16 bytes; scale,
 *     max and index arrays 4 bytes; workspace 256 bytes.
 *   - Non-finite inputs give unspecified (but memory-safe) results.
 */
#ifndef MTPD_H
#define MTPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MTPD_OK = 0,
    MTPD_ERR_NULL = 1,      /* a required pointer is NULL */
    MTPD_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
    MTPD_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
    MTPD_ERR_ALIAS = 4,     /* an output overlaps an input or another output */
    MTPD_ERR_WORKSPACE = 5, /* workspace missing or smaller than mtpd_workspace_bytes */
    MTPD_ERR_HIP = 6        /* the HIP runtime refused a launch or query */
} mtpd_status;

/* Packed FP8 activation ("QuantizedActivation"): codes [rows][cols] OCP
 * E4M3FN, scales [rows][cols/128] fp32 dequant multipliers.  cols % 128 == 0. */
typedef struct {
    uint8_t *codes;
    float *scales;
    int64_t rows;
    int64_t cols;
} mtpd_qact;

/* Shared FP8 LM head (or this GPU's vocab shard of it): codes [V][H] OCP
 * E4M3FN, K contiguous; scales [V/128][H/128] fp32, one per 128x128 block. */
typedef struct {
    const uint8_t *codes;
    const float *scales;
    int64_t V;
    int64_t H;
} mtpd_fp8_weight;

/*
 * Residual add + RMSNorm + dual output
 * ("Reuse packed FP8 logits inputs", Purpose; fp32 accumulation per
 * "Fuse the MTP trailing all-reduce; local-argmax draft tokens", Accuracy).
 *
 *   s = f32(hidden) + f32(residual)                      per element
 *   rstd = 1 / sqrt(sum(s^2) / H + eps)                  sum accumulated in fp32
 *   y = s * rstd * norm_weight                           fp32, not rounded
 *   out_hidden = RNE_bf16(y)                             the recycled hidden
 *   per 128-column block b of each row:
 *     scale_b = RN_f32(max|y| / 448)                     dequant multiplier
 *     code    = E4M3(RN_f32(y / scale_b)), clamped to +-448, ties to even
 *     (scale_b == 0 gives scale 0 and all codes 0x00)
 *
 * hidden, residual: [M][H] bf16.  norm_weight: [H] f32.  eps: added to the
 * mean square (inside the square root).  out_hidden: [M][H] bf16.  out_act:
 * rows == M, cols == H; its codes and scales are written.
 */
mtpd_status mtpd_norm_quant(const uint16_t *hidden, const uint16_t *residual,
                            const float *norm_weight, float eps, int64_t M, int64_t H,
                            uint16_t *out_hidden, const mtpd_qact *out_act, void *stream);

/*
 * Block-scaled FP8 LM head fused with a greedy local argmax
 * ("Reuse packed FP8 logits inputs", Purpose and Dependencies;
 * "Fuse the MTP trailing all-reduce; local-argmax draft tokens", Summary).
 *
 * For output row i, with a = row_index ? row_index[i] : i:
 *   z[v] = sum_b act.scales[a][b] * w.scales[v/128][b] *
 *          sum_{k in block b} dec(act.codes[a][k]) * dec(w.codes[v][k])
 *   out_idx[i] = the lowest v in [0, V) attaining the largest fp32 z[v]
 *                (+0 and -0 compare equal); out_max[i] = that z, in fp32.
 * The logits z are never written to memory.  out_idx is local to this
 * weight (a vocab shard's caller adds the shard offset).
 *
 * act: rows >= 1, cols == w->H.  row_index: [n_rows] int32 rows of act, or
 * NULL for rows 0..n_rows-1 (then n_rows <= act->rows); its values must lie
 * in [0, act->rows) and are not checked on the device.  out_max: [n_rows]
 * f32.  out_idx: [n_rows] int32.
 * workspace: device memory of at least mtpd_workspace_bytes(n_rows) bytes,
 * ZERO-FILLED before its first use; every call that runs to completion
 * leaves it zero-filled again.  Calls that share a workspace must not
 * overlap in time; after a call that did not complete, zero it again.
 */
mtpd_status mtpd_fp8_lmhead_argmax(const mtpd_qact *act, const int32_t *row_index, int64_t n_rows,
                                   const mtpd_fp8_weight *w, float *out_max, int32_t *out_idx,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole draft tail for M rows: mtpd_norm_quant followed by
 * mtpd_fp8_lmhead_argmax on every row of the packed activation it produced
 * (row_index NULL).  This is the producer/consumer pair of
 * "[Quant][MTP] Reuse packed FP8 logits inputs", Purpose (the MTP layer
 * returns the packed activation and the bf16 hidden; the shared LM head
 * consumes the packed activation as it is) closed by the local greedy
 * argmax of "[Spec Decode][Perf] Fuse the MTP trailing all-reduce;
 * local-argmax draft tokens", Summary.  Same arguments, layouts, workspace
 * contract and results as the two calls in sequence; w->H must equal H.
 * One row with H <= 8192 runs as a single fused launch whose recycled
 * hidden, codes and scales are bit-identical to the two-launch path.
 */
mtpd_status mtpd_draft_tail(const uint16_t *hidden, const uint16_t *residual,
                            const float *norm_weight, float eps, int64_t M, int64_t H,
                            const mtpd_fp8_weight *w, uint16_t *out_hidden, const mtpd_qact *out_act,
                            float *out_max, int32_t *out_idx,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * mtpd_draft_tail for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments without the workspace, the
 * same kernels and bit-identical results.  The argmax keys and arrival
 * counters live in a device array inside the library, 528640 bytes per GPU
 * (held until the process ends), which covers M <= 65536; a larger M returns
 * MTPD_ERR_WORKSPACE and launches nothing.  The first call on a device
 * clears that array with a fill kernel on `stream`; every completed call
 * leaves it clear again.  The array is shared by every call on the same GPU:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * give wrong results; serialize them.  Never calls hipMalloc or hipFree.
 */
mtpd_status mtpd_draft_tail_noalloc(const uint16_t *hidden, const uint16_t *residual,
                                    const float *norm_weight, float eps, int64_t M, int64_t H,
                                    const mtpd_fp8_weight *w, uint16_t *out_hidden,
                                    const mtpd_qact *out_act, float *out_max, int32_t *out_idx,
                                    void *stream);

/*
 * mtpd_norm_quant with the MTP layer's trailing all-reduce folded in
 * ("Fuse the MTP trailing all-reduce; local-argmax draft tokens", Summary:
 * all-reduce and RMSNorm as one fused step; Accuracy: fp32 accumulation).
 * The norm input is the sum of the row-parallel partial outputs of the
 * layer's last projection plus the residual:
 *
 *   s = f32(partials[0]) + f32(partials[1]) + ... + f32(partials[P-1])
 *       + f32(residual)      accumulated in fp32, left to right
 *
 * and everything after s is exactly mtpd_norm_quant's (same outputs, same
 * rounding); with n_partials == 1 the results are bit-identical to
 * mtpd_norm_quant(partials[0], residual, ...).
 *
 * partials: a HOST array of n_partials device pointers, each [M][H] bf16 (on
 * one GPU they stand in for the peers' buffers a one-shot all-reduce reads;
 * moving data between GPUs is not part of this call).  1 <= n_partials <= 16.
 * The other arguments are mtpd_norm_quant's; no output may overlap a partial.
 */
mtpd_status mtpd_allreduce_norm_quant(const uint16_t *const *partials, int64_t n_partials,
                                      const uint16_t *residual, const float *norm_weight, float eps,
                                      int64_t M, int64_t H, uint16_t *out_hidden, const mtpd_qact *out_act,
                                      void *stream);

/*
 * Vocab-parallel combine of per-shard greedy argmaxes
 * ("Fuse the MTP trailing all-reduce; local-argmax draft tokens", Summary:
 * each GPU's local argmax over its vocab slice replaces the gather of
 * full-vocab logits).  Shard s covers global vocab rows shard_offset[s] ..
 * and returned local pairs (local_max[s][i], local_idx[s][i]) from
 * mtpd_fp8_lmhead_argmax.  For each row i:
 *   out_idx[i] = the lowest global index shard_offset[s] + local_idx[s][i]
 *                among the shards whose local_max[s][i] is the largest
 *                (+0 and -0 compare equal);
 *   out_max[i] = that maximum (-0 is returned as +0).
 * When the shards tile [0, V) this equals the full-vocab greedy argmax.
 *
 * local_max: [n_shards][n_rows] f32, local_idx: [n_shards][n_rows] int32,
 * device memory, row-major.  shard_offset: HOST array of n_shards values in
 * [0, 2^31 - 128]; every offset + local index must stay below 2^31 (not
 * checked on the device).  out_max: [n_rows] f32, out_idx: [n_rows] int32.
 * 1 <= n_shards <= 64; n_rows == 0 launches nothing.  No workspace.
 */
mtpd_status mtpd_argmax_combine(const float *local_max, const int32_t *local_idx,
                                const int64_t *shard_offset, int64_t n_shards, int64_t n_rows,
                                float *out_max, int32_t *out_idx, void *stream);

/*
 * Vocab-parallel combine of per-shard top-k lists (the same passages as
 * mtpd_argmax_combine; "feat(glm52): add checkpoint-native MTP speculative
 * decoding", Accuracy, compares top-8 and top-32 sets).  Shard s covers
 * global vocab rows shard_offset[s] .. and returned, per row i, its list
 * (local_val[s][i][0..k), local_idx[s][i][0..k)) from mtpd_fp8_lmhead_topk:
 * descending values, equal values in ascending index order.  For each row:
 *   out_idx[i][0..k) = the global indices shard_offset[s] + local_idx[s][i][j]
 *                      of the k largest values over all shards' lists, in
 *                      descending value, equal values (+0 and -0 equal) in
 *                      ascending global index;
 *   out_val[i][e]    = that value (-0 returned as +0).
 * When the shards tile [0, V), hold disjoint vocab rows and each returned its
 * own top-k, this equals the full-vocab top-k.  The lists must be sorted as
 * described (the combine merges them; unsorted lists give a wrong result,
 * not an error).
 *
 * local_val: [n_shards][n_rows][k] f32, local_idx: [n_shards][n_rows][k]
 * int32, device memory, row-major.  shard_offset: HOST array of n_shards
 * values in [0, 2^31 - 128]; every offset + local index must stay below
 * 2^31 (not checked on the device).  out_val, out_idx: [n_rows][k].
 * 1 <= n_shards <= 64, 1 <= k <= 32; n_rows == 0 launches nothing.  No
 * workspace.
 */
mtpd_status mtpd_topk_combine(const float *local_val, const int32_t *local_idx,
                              const int64_t *shard_offset, int64_t n_shards, int64_t n_rows,
                              int64_t k, float *out_val, int32_t *out_idx, void *stream);

/*
 * Block-scaled FP8 LM head fused with a greedy local top-k
 * ("Reuse packed FP8 logits inputs", Purpose and Dependencies, for the
 * logits; "feat(glm52): add checkpoint-native MTP speculative decoding",
 * Accuracy, where draft and reference distributions are compared by their
 * top-8 and top-32 sets).
 *
 * With z as in mtpd_fp8_lmhead_argmax, for output row i:
 *   out_idx[i][0..k) = the k vocab rows of largest fp32 z, in descending
 *                      order of z, equal values in ascending index order
 *                      (+0 and -0 equal); out_val[i][e] = that z in fp32
 *                      (-0 returned as +0).  k == 1 gives the argmax.
 * Logits are never written; per pass of at most 64 rows the streaming
 * kernel writes one sorted candidate list of k keys per row for each of its
 * waves (at most V/32 lists) to the workspace and a second launch selects
 * from them.  More than 64 rows run as several passes, each streaming the
 * whole weight.
 *
 * act, row_index, n_rows, w: as for mtpd_fp8_lmhead_argmax; additionally
 * w->H <= 8192 and act->rows * w->H <= 2^32.  1 <= k <= 32.  out_val:
 * [n_rows][k] f32, out_idx: [n_rows][k] int32.  workspace: at least
 * mtpd_topk_workspace_bytes(n_rows, w->V, k) bytes of device memory, 256-byte
 * aligned, any contents (nothing needs to be zero).
 */
mtpd_status mtpd_fp8_lmhead_topk(const mtpd_qact *act, const int32_t *row_index, int64_t n_rows,
                                 const mtpd_fp8_weight *w, int64_t k, float *out_val, int32_t *out_idx,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes mtpd_fp8_lmhead_topk needs (a multiple of 256; 0 for
 * n_rows <= 0 or sizes it does not take). */
size_t mtpd_topk_workspace_bytes(int64_t n_rows, int64_t V, int64_t k);

/* Bytes of workspace mtpd_fp8_lmhead_argmax / mtpd_draft_tail need for
 * n_rows output rows (a multiple of 256; 0 for n_rows <= 0 or above 2^24). */
size_t mtpd_workspace_bytes(int64_t n_rows);

/* Static name of a status code ("MTPD_OK", ...); "MTPD_UNKNOWN" otherwise. */
const char *mtpd_status_name(mtpd_status s);

/* Detail of the first failure on the calling thread since the last
 * mtpd_clear_error (empty string if none).  The first failure is kept, not
 * the latest, so the root cause survives the errors it provokes (the
 * practice "feat(glm52): add checkpoint-native MTP speculative decoding",
 * Description, follows for its own failures).  The pointer stays valid until
 * the next mtpd_clear_error on this thread. */
const char *mtpd_last_error(void);
void mtpd_clear_error(void);

/* Diagnostics: the kernel (and launch shape) mtpd_fp8_lmhead_argmax would
 * run for these sizes, e.g. "lmhead_decode_kernel<4,2,2> grid=1184x256",
 * as a static thread-local string; "" if the sizes are invalid.  Makes no
 * HIP call except a one-time query of the current device's CU count. */
const char *mtpd_lmhead_plan(int64_t n_rows, int64_t V, int64_t H);

/* Diagnostics: the kernel launches mtpd_draft_tail would make for M rows,
 * e.g. "draft_tail1_kernel grid=1184x256" (one fused launch, M = 1) or
 * "norm_quant_kernel<3> grid=64x256 + lmhead_stream_rows_kernel<4,2,4,3>
 * grid=1184x256"; same string rules as mtpd_lmhead_plan. */
const char *mtpd_draft_tail_plan(int64_t M, int64_t V, int64_t H);

/*
 * Launch-plan override, for tuning sweeps and tests only: pins the kernel
 * (or launch shape) the dispatcher picks, so that every compiled shape can be
 * checked against the same results.  Results stay within the documented
 * tolerances under any setting; only the speed and the fp32 summation order
 * change.  Process-wide, read by the host-side dispatch of every later call:
 * set it only while no call of this library is being made on any thread.
 *
 *   key               value
 *   "lmhead_kernel"   "generic" (the generic tiled kernel only) or "decode"
 *                     (no weight-streaming kernels), NULL for automatic
 *   "lmhead_tile"     "nt,s,d"       generic kernel shape
 *   "lmhead_stream"   "nt,d"         weight-streaming kernel shape
 *   "lmhead_rows"     "nt,nw,d"      shared-activation streaming kernel shape
 *   "lmhead_decode"   "nt,d"         register-staged decode kernel shape
 *   "lmhead_kouter"   "0" (never) or "nt,nw,d,tmax" (only that shape)
 *   "lmhead_gemm"     "n"            compute-regime kernel variant (0 automatic)
 *   "draft_tail"      "split" (one row runs as two launches, not fused)
 *   "norm_quant"      "wave" (a wavefront per row, H <= 8192) or
 *                     "workgroup" (a workgroup per row, the default)
 *   "device_cus"      "n"            size persistent grids for n CUs
 *
 * A NULL value clears that key; a NULL key clears every key.  Returns
 * MTPD_ERR_SHAPE (and changes nothing) for an unknown key or a value that
 * does not parse.
 */
mtpd_status mtpd_set_plan_override(const char *key, const char *value);

/* ABI version: bumped when any declaration above changes. */
int mtpd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTPD_H */
