/*
 * q4rac -- NVFP4 W4A4 GEMM with Residual Activation Compensation on MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer unless marked (host); every
 * call enqueues its work asynchronously on `stream` (a hipStream_t passed as
 * void*, NULL = the default stream) and returns after launching.  The caller
 * owns all memory: the library never allocates or frees device memory; calls
 * that need scratch memory take a caller-provided `workspace` whose minimum size
 * the matching *_workspace_size() function returns.  Every argument check runs
 * on the host before any launch, so a call that returns an error has enqueued
 * nothing and written nothing.  Errors are returned as q4_status_t codes;
 * q4_last_error() returns a thread-local message for the last failure in the
 * calling thread.  Device-side faults surface at the caller's next
 * synchronisation.  Calls are stateless and thread-safe when they use distinct
 * workspaces and outputs.
 *
 * Sizes: rows, M, N and T * topk below 2^31; channels of a quantized tensor and
 * the GEMM reduction length K (MoE: H and F) at most 2^24 (larger ones are
 * refused with Q4_ESHAPE).  Within those limits every shape runs; the fastest
 * kernels address a tile's operands with 32-bit offsets and are used only
 * where those fit (tiled scale records of at most 4 GiB per operand, a
 * gathered MoE activation operand of at most 4 GiB, an expert weight matrix
 * of at most 4 GiB of codes), other shapes run on kernels with 64-bit
 * addressing and give the same results.
 *
 * Alignment: tensor scales, logits, routing weights and index arrays need 4-byte
 * alignment, channel scores 8-byte; every other device pointer (activations,
 * codes, scales, outputs, workspaces) must be 16-byte aligned.  Inputs must be
 * finite (bf16 activations and weights, fp32 logits); this is documented, not
 * checked.
 *
 * Method: QUADS (arXiv 2607.15810), section 2.2 paragraph "FP4" for the NVFP4
 * format, section 3.3 Eq. 20-24 for the residual compensation.  Layouts:
 *
 *   x        bf16 [rows][cols] row-major; cols is the channel (reduction) axis.
 *   codes    uint8 [rows][cols/2]: element 2i in the low nibble, 2i+1 in the
 *            high nibble; nibble = E2M1 magnitude code (0..7 for
 *            0,0.5,1,1.5,2,3,4,6) | 8 * sign bit of x.
 *   scales   NVFP4: uint8 [rows][cols/16], E4M3 (bias 7, no infinities, 0x7F
 *            unused) block scale of sixteen consecutive elements of a row.
 *            MXFP4: uint8 [rows][cols/32], E8M0 exponent byte e + 127.
 *   tensor   NVFP4: fp32 per-tensor scale s_t; value = code * block * s_t.
 *
 * Quantization rule (the plain reading of the page; each "nearest" is decided
 * on the exact real quotient):
 *   s_t = RN32(amax / 2688) (6 * 448: largest E2M1 magnitude times the largest
 *         E4M3 value), 1 for an all-zero tensor, or the caller's value;
 *   sb  = E4M3 nearest to amax_block / (6 s_t), ties to the even code,
 *         saturating at 448;
 *   c   = E2M1 magnitude nearest to |x| / (sb s_t), ties to the even code,
 *         saturating at 6, zero when sb == 0;
 *   MXFP4: block of 32, scale 2^e, e = floor(log2 amax_block) - 2 clamped to
 *         [-127, 127] (byte 0 for an all-zero block), c nearest to |x| / 2^e.
 *   residual r = RN32(x - dequant(x)) (the negated Eq. 20 error);
 *   channel score_j = sum_i r_ij^2 (Eq. 23 squared): the exact fp64 squares
 *         summed in fp64 in a fixed order (so a call is deterministic), which
 *         is within (rows - 1) * 2^-53 relative of the exact sum;
 *   channel set S = the topk channels of largest score, ties to the smaller
 *         channel, listed in ascending channel order (Eq. 24, absolute k).
 *
 * Status words: calls that take a device channel set or device expert indices
 * also take `status`, an optional device int32 [1].  When given, the call
 * writes Q4_OK there, or Q4_EINVAL if those device inputs break their
 * contract (the call then takes the documented safe path instead of reading
 * out of bounds or double counting).  It is written in stream order, like the
 * outputs.
 */
#ifndef Q4RAC_H
#define Q4RAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  Q4_OK = 0,
  Q4_EINVAL = 1,        /* null pointer, bad enum, bad k                         */
  Q4_ESHAPE = 2,        /* dimension not supported (see each call)               */
  Q4_EALIGN = 3,        /* pointer not 16-byte aligned                            */
  Q4_EWORKSPACE = 4,    /* workspace smaller than *_workspace_size()             */
  Q4_EUNSUPPORTED = 5,  /* format / option combination not provided              */
  Q4_EHIP = 6           /* a HIP launch or runtime call failed                   */
} q4_status_t;

typedef enum { Q4_NVFP4 = 0, Q4_MXFP4 = 1 } q4_format_t;
typedef enum { Q4_OUT_F32 = 0, Q4_OUT_BF16 = 1 } q4_dtype_t;

#define Q4_MAX_TOPK 1024

/* (host) message for the last non-OK status returned in this thread. */
const char *q4_last_error(void);
/* (host) library ABI version (major * 100 + minor). */
int32_t q4_version(void);

/* ---------------------------------------------------------------- quantizer
 * Workspace bytes needed by nvfp4_quantize / mxfp4_quantize for this shape
 * (fp64 partial channel sums, the amax word and the top-k scratch). */
size_t q4_quantize_workspace_size(int64_t rows, int64_t cols, int32_t fmt);

/* Online NVFP4 activation quantization with per-channel residual statistics
 * (QUADS section 2.2 "FP4"; section 3.3 Eq. 20, 23, 24).
 *   x               bf16 [rows][cols]; rows >= 0, cols > 0, cols % 16 == 0.
 *   tensor_scale_in fp32 [1] or NULL.  NULL: s_t is computed from the tensor's
 *                   amax inside the call.  Otherwise its value (positive,
 *                   finite, normal) is used as s_t.
 *   codes           uint8 [rows][cols/2] (out).   scales uint8 [rows][cols/16] (out).
 *   tensor_scale_out fp32 [1] (out): the s_t used.
 *   chan_score      fp64 [cols] (out) or NULL: sum of squared residuals.
 *   topk            0 <= topk <= min(cols, Q4_MAX_TOPK); 0 skips the selection.
 *   chan_idx        int32 [topk] (out), ascending channel indices; NULL iff topk == 0.
 * rows == 0 is valid: s_t = 1 (or the supplied value), scores are 0 and the
 * selection is channels 0..topk-1. */
q4_status_t nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols,
                           const float *tensor_scale_in, uint8_t *codes, uint8_t *scales,
                           float *tensor_scale_out, double *chan_score, int32_t topk,
                           int32_t *chan_idx, void *workspace, size_t workspace_bytes,
                           void *stream);

/* MXFP4 variant (the open-standard MXFP4 with power-of-two block scales named
 * by the Rollout-ResQ abstract on the listing page thelatestinai.com,
 * papers/2607.15810; block rule of the OCP MX format): cols % 32 == 0; scales
 * uint8 [rows][cols/32] E8M0; no tensor scale.  Residual statistics and
 * selection as nvfp4_quantize (QUADS section 3.3, Eq. 20, 23, 24). */
q4_status_t mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *codes,
                           uint8_t *scales, double *chan_score, int32_t topk, int32_t *chan_idx,
                           void *workspace, size_t workspace_bytes, void *stream);

/* nvfp4_quantize for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, kernels and results as
 * nvfp4_quantize, minus the workspace: the scratch comes from a static device
 * array of nvfp4_quantize_noalloc_max_scratch() bytes (24 MiB) that each GPU
 * the library runs on holds until the process ends.  The call allocates
 * nothing.  A shape whose scratch (q4_quantize_workspace_size) exceeds that
 * maximum returns Q4_EWORKSPACE before any launch.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams
 * or host threads without ordering between them) race, so serialize them.
 * Nothing in the array needs to start at zero. */
size_t nvfp4_quantize_noalloc_max_scratch(void);
q4_status_t nvfp4_quantize_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                   const float *tensor_scale_in, uint8_t *codes,
                                   uint8_t *scales, float *tensor_scale_out, double *chan_score,
                                   int32_t topk, int32_t *chan_idx, void *stream);

/* Trainer-side weight fake quantization (QUADS section 3.2, Eq. 12, and the
 * alignment of Eq. 16: the trainer's weight quantize-dequantize must use the
 * same block layout and the same rounding as the rollout kernels, so both
 * sides compute with one discretized weight):
 *   y = c * sb * s_t of nvfp4_quantize(x) (the same kernels, so the codes,
 *       scales and s_t are those nvfp4_quantize gives), rounded once to fp32
 *       or to bf16 (y_dtype).
 *   x, rows, cols, tensor_scale_in as nvfp4_quantize; y [rows][cols];
 *   tensor_scale_out fp32 [1] (out) or NULL.
 * The backward of the page's straight-through estimator (Eq. 13) is the
 * identity on the gradient and needs no kernel. */
size_t nvfp4_qdq_workspace_size(int64_t rows, int64_t cols);
q4_status_t nvfp4_qdq(const uint16_t *x, int64_t rows, int64_t cols, const float *tensor_scale_in,
                      void *y, int32_t y_dtype, float *tensor_scale_out, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Channel selection alone (section 3.3 Eq. 24) from fp64 scores [cols]:
 * the topk largest, ties to the smaller index, written ascending to chan_idx. */
size_t q4_select_workspace_size(int64_t cols);
q4_status_t q4_select_channels(const double *chan_score, int64_t cols, int32_t topk,
                               int32_t *chan_idx, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Residual gather (section 3.3 Eq. 21 on the selected channels):
 * R[i][t] = bf16_RNE(r[i][S_t]) for t < k, and 0 for k <= t < ld_r, where r is
 * the fp32 residual of x against its quantized form (codes/scales/tensor scale;
 * tensor_scale must be NULL for MXFP4).  R is bf16 [rows][ld_r], ld_r >= k.
 * chan_idx must hold k ascending, unique channels in [0, cols); a set that
 * does not gathers nothing (R all zero) and sets *status to Q4_EINVAL. */
q4_status_t q4_residual_gather(int32_t fmt, const uint16_t *x, int64_t rows, int64_t cols,
                               const uint8_t *codes, const uint8_t *scales,
                               const float *tensor_scale, const int32_t *chan_idx, int32_t k,
                               uint16_t *R, int64_t ld_r, int32_t *status, void *stream);

/* ---------------------------------------------------------------- GEMM
 * W4A4 GEMM (QUADS section 3.3, the native W4A4 product that Eq. 22's remark
 * keeps on the FP4 path):
 *   Y[i][j] = s_A s_W sum_k (c sb)_A[i][k] (c sb)_W[j][k]
 * A is M x K (activations), W is N x K (weights, "out x in"); both in `fmt`
 * with the layouts above.  a_tensor_scale / w_tensor_scale: fp32 [1] for
 * NVFP4, NULL for MXFP4.  Y is [M][N] fp32 or bf16 (round to nearest even).
 * Shapes: M >= 0, N >= 0, K > 0 with K % 32 == 0. */
q4_status_t w4a4_gemm(int32_t fmt, int64_t M, int64_t N, int64_t K, const uint8_t *a_codes,
                      const uint8_t *a_scales, const float *a_tensor_scale,
                      const uint8_t *w_codes, const uint8_t *w_scales,
                      const float *w_tensor_scale, void *Y, int32_t y_dtype, void *stream);

/* W4A4 GEMM with Residual Activation Compensation (section 3.3 Eq. 21-22):
 *   Y = W4A4(A, W) + sum_{t<k} R[i][t] W_hi[j][S_t]
 * with R the bf16 residual of x on the channel set S (q4_residual_gather) and
 * W_hi the bf16 weight.  The compensation is accumulated into the same fp32
 * tile as the W4A4 product: for NVFP4 as fp16 MFMA steps on R 2^-e_A (exact)
 * and W_hi / (s_W f_A) (W_hi times the fp32 reciprocal of s_W f_A, rounded
 * to fp16: relative error at most 2^-11 + 2^-21; s_A = f_A 2^e_A) into the
 * unscaled sum, then s_A s_W multiplies both; for MXFP4 as bf16 steps.  The
 * compensation term therefore carries that relative rounding, which matters
 * only where it is large against the output (blocks saturated under a
 * supplied tensor scale).  Range (documented, not checked): |r| / s_A and |W_hi| / s_W below
 * 2^15 (with tensor scales taken from the operands' own amax they are at
 * most 448 and 2688).  s_A s_W itself may be as small as the fp32 range
 * allows: it is applied as mantissa and exponent, so only a result that is
 * itself subnormal loses bits.
 *   x       bf16 [M][K], the activation that produced A.
 *   w_hi_t  bf16 [K][N]: the transposed bf16 weight (channel-major), so the
 *           selected rows S_t are contiguous.
 *   chan_set int32 [k] ascending unique channels in [0, K);
 *           0 <= k <= min(K, Q4_MAX_TOPK).  Checked on the device: a set
 *           that is not ascending, unique and in range adds no compensation
 *           (Y is then exactly w4a4_gemm) and sets *status to Q4_EINVAL.
 *   status  int32 [1] (out, device) or NULL: Q4_OK / Q4_EINVAL as above.
 * k == 0 gives exactly w4a4_gemm.
 * Workspace: R and the selected weight columns (when k > 0) and, for NVFP4
 * with K % 128 == 0, re-laid-out fp16 copies of both operands' block scales
 * that the large-tile kernel reads; with k == 0 the workspace is optional (a
 * null or smaller one selects the kernel that reads the scales in place).
 * Results are identical either way. */
size_t rac_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t k);
q4_status_t rac_gemm(int32_t fmt, int64_t M, int64_t N, int64_t K, const uint16_t *x,
                     const uint8_t *a_codes, const uint8_t *a_scales,
                     const float *a_tensor_scale, const uint8_t *w_codes,
                     const uint8_t *w_scales, const float *w_tensor_scale,
                     const uint16_t *w_hi_t, const int32_t *chan_set, int32_t k, void *Y,
                     int32_t y_dtype, void *workspace, size_t workspace_bytes, int32_t *status,
                     void *stream);

/* Page-literal compensation (QUADS section 3.3, Eq. 20-21), NVFP4 only.  The
 * quantization error dX = dequant(A) - x is quantized as an activation of its
 * own: carried as bf16 (dX = bf16(RN32(dequant - x))), tensor scale
 * s_R = RN32(amax|dX| / 2688) (1 if dX is all zero), E4M3 block scales and
 * E2M1 codes by the quantization rule above.  It is masked to the channel set
 * S after quantization, and the corrected activation multiplies the NVFP4
 * weight (no bf16 weight is needed):
 *   Y = ( dequant(A) - M_S * dequant(Q(dX)) ) W_dequant^T
 *     = s_A s_W sum_K d_A d_W - s_R s_W sum_{t<k} (c sb)_dX[i][S_t] (c sb)_W[j][S_t].
 * Both factors of the second sum are exact in fp16; it runs as extra fp16
 * MFMA steps into the same fp32 tile.
 *   x, A, W, chan_set, k, Y, y_dtype, status as rac_gemm (A and W NVFP4; an
 *           invalid channel set adds no compensation and reports Q4_EINVAL).
 *   resid_tensor_scale_out fp32 [1] (out) or NULL: s_R, written when M, N and
 *           k are all > 0.
 * k == 0 gives exactly w4a4_gemm.  Range (documented, not checked): the W4A4
 * sum is carried scaled by s_A / s_R on one path and the compensation by
 * s_R / s_A on the other, so s_R / s_A must lie in [2^-90, 2^90].  With s_A
 * computed from the tensor's own amax it is at most 1/6 (or dX is all zero,
 * which is harmless); it falls below 2^-90 only for a tensor whose largest
 * quantization error is below about 2^-90 of its largest element.
 * Workspace (rac_gemm_eq21_workspace_size): at offset 0 the fp16 matrix
 * R' [M][kp] = (c sb) of Q(dX) on S (0 past k; exact in fp16), kp = k rounded
 * up to 32, then the weight factor [N][kp], the amax partials, s_R and the
 * scale records. */
size_t rac_gemm_eq21_workspace_size(int64_t M, int64_t N, int64_t K, int32_t k);
q4_status_t rac_gemm_eq21(int64_t M, int64_t N, int64_t K, const uint16_t *x,
                          const uint8_t *a_codes, const uint8_t *a_scales,
                          const float *a_tensor_scale, const uint8_t *w_codes,
                          const uint8_t *w_scales, const float *w_tensor_scale,
                          const int32_t *chan_set, int32_t k, void *Y, int32_t y_dtype,
                          float *resid_tensor_scale_out, void *workspace,
                          size_t workspace_bytes, int32_t *status, void *stream);

/* ---------------------------------------------------------------- MoE
 * The QUADS page compensates the activations of MoE expert projections: its
 * profiled site is the W13 (gate/up) input, section 3.3 "Online per-channel
 * selection", and Figure 4b compares layer-wise MoE outputs.  It does not
 * spell out the expert block; the calls below are the standard top-k SwiGLU
 * expert layer.
 *
 * Router: for each token the topk experts of largest logit (ties to the
 * smaller expert), highest first, and their weights softmax(selected logits).
 * logits fp32 [T][E]; 1 <= topk <= min(E, 16); E <= 1024.  topk_idx int32
 * [T][topk], topk_w fp32 [T][topk].  A NaN logit ranks below every number
 * (every token still gets topk distinct experts in [0, E)). */
q4_status_t q4_moe_route(const float *logits, int64_t T, int32_t E, int32_t topk,
                         int32_t *topk_idx, float *topk_w, void *stream);

/* Token sort for the grouped GEMM of the W13 site (section 3.3): routed rows
 * (t, s) ordered by (expert, t, s), a stable counting sort.
 * perm int32 [T*topk]: perm[r] = t*topk + s of sorted row r; offsets int32
 * [E+1] (offsets[e] = first sorted row of expert e).  workspace:
 * q4_moe_sort_workspace_size.  An index outside [0, E) is invalid: it is
 * sorted as expert 0 (nothing is written out of bounds) and *status (device
 * int32 [1], optional) is set to Q4_EINVAL. */
size_t q4_moe_sort_workspace_size(int64_t T, int32_t E, int32_t topk);
q4_status_t q4_moe_sort(const int32_t *topk_idx, int64_t T, int32_t E, int32_t topk,
                        int32_t *perm, int32_t *offsets, void *workspace,
                        size_t workspace_bytes, int32_t *status, void *stream);

/* Weight preparation (offline).
 * q4_transpose_bf16: out[c][b][r] = in[b][r][c] for `batch` stacked
 *   [rows][cols] bf16 matrices (one matrix: out[c][r] = in[r][c]), so the
 *   output is channel-major with the matrices interleaved, [cols][batch][rows].
 *   Used to build W_hi^T: the batch's rows of one channel are contiguous, and
 *   a gather of the selected channels reads a few contiguous runs.
 * q4_moe_pack_w13: the logical W13 of each expert, [2F][H] with gate rows
 *   0..F-1 and up rows F..2F-1, is re-ordered into groups of 32 rows
 *   [gate 32g..32g+31, up 32g..32g+31] for g = 0..F/32-1 (F % 32 == 0); the
 *   grouped GEMM's SwiGLU epilogue then finds a gate column and its up column
 *   in the same tile.  Row order commutes with quantization (blocks run along H). */
q4_status_t q4_transpose_bf16(const uint16_t *in, int64_t batch, int64_t rows, int64_t cols,
                              uint16_t *out, void *stream);
q4_status_t q4_moe_pack_w13(const uint16_t *w13, int32_t E, int32_t F, int32_t H,
                            uint16_t *out, void *stream);

/* Scale records of stacked weights (offline), laid out per 128-column chunk
 * as [batch][K/128][rows_pad][record], rows_pad = rows rounded up to 256
 * (rows past `rows` zero), so that a tile's rows of one chunk are contiguous.
 *   fmt Q4_NVFP4: the E4M3 block scales (one per 16 elements, QUADS section
 *     2.2 "FP4" and the NVFP4 format pages) of operands [rows][K/16], twice:
 *     first widened to fp16 (exact, subnormal scales included), a 16-byte
 *     record holding the eight scales of one row and chunk with its four
 *     dwords in an order that spreads a tile's LDS reads over the banks (read
 *     by the 256 x 256 grouped GEMM); then as raw bytes, an 8-byte record
 *     holding the same eight scales in block order (read by the grouped GEMM
 *     of decode-shaped layers, which streams the weights: half the bytes).
 *     Size batch * (K/128) * rows_pad * 24.
 *   fmt Q4_MXFP4: the E8M0 scales (one per 32 elements) of operands
 *     [rows][K/32]: a 4-byte record holds the four of one row and chunk.
 * Derived data only: a grouped GEMM given the records computes exactly what
 * it computes from the raw scales.  K % 128 == 0 (Q4_ESHAPE otherwise); out
 * must hold q4_scale_records_size bytes (Q4_EWORKSPACE); out is caller-owned. */
size_t q4_scale_records_size(int32_t fmt, int64_t batch, int64_t rows, int64_t K);
q4_status_t q4_scale_records(int32_t fmt, const uint8_t *scales, int64_t batch, int64_t rows,
                             int64_t K, uint8_t *out, size_t out_bytes, void *stream);

/* Token-sorted grouped W4A4 + RAC SwiGLU expert layer: the compensation of
 * QUADS section 3.3 (Eq. 21-24) at both activation sites of the expert block,
 * the W13 input (the page's profiled site) and the W2 input.
 *   tokens     bf16 [T][H]; H % 32 == 0 (MXFP4: % 32; NVFP4 GEMM: % 32).
 *   topk_idx, topk_w: routing as produced by q4_moe_route.
 *   w13_*      stacked packed W13 of all experts: rows E*2F (q4_moe_pack_w13
 *              order), cols H; w13_tensor_scales fp32 [E] (NVFP4) or NULL.
 *   w2_*       stacked W2: rows E*H, cols F; w2_tensor_scales fp32 [E] or NULL.
 *   w13_hi_t   bf16 [H][E][2F]: q4_transpose_bf16 of the packed bf16 W13
 *              (the experts' transposes, channel-major and interleaved).
 *   w2_hi_t    bf16 [F][E][H]:  q4_transpose_bf16 of the bf16 W2.
 *              Both may be NULL when rac_k == 0.
 *   w13_scale_records, w2_scale_records: NULL, or the q4_scale_records (in
 *              the layer's format) of w13_scales (batch E, rows 2F, K = H) and
 *              of w2_scales (batch E, rows H, K = F), which must be those
 *              scales' records (not checked).  Where the shape allows (H and F
 *              multiples of 128; prefill-sized T * topk also needs them at
 *              least 512) the grouped GEMMs then read the records instead of
 *              the raw scales; results are the same.
 *   h_tensor_scale: NULL, or (NVFP4 only) device fp32 [1]: h's tensor scale
 *              supplied by the caller (delayed scaling, e.g. an earlier step's
 *              s_h) instead of RN32(amax(h) / 2688): the quantizer runs on h
 *              with this scale and no amax pass.  Blocks whose amax exceeds
 *              2688 s_h saturate (E4M3 scale 448, codes +-6), as the format
 *              defines.  moe_w4a4_grouped_gemm_ex can instead quantize h inside
 *              the W13 GEMM (Q4_MOE_FUSE_H_QUANT).
 *   rac_k      channels compensated at each of the two activation sites.
 *   Y          [T][H] fp32 or bf16: y_t = sum_s p_ts out_(t,s), slots in order,
 *              summed in fp32.  The expert rows out_(t,s) are kept in Y's type:
 *              with a bf16 Y each is rounded to bf16 (nearest even) first.
 * Steps: sort; quantize tokens (one s_t, one selection over T rows); W13 RAC
 * GEMM over sorted rows with the SwiGLU epilogue h = bf16(silu(g) * u); quantize
 * h over all T*topk sorted rows (one s_t, one selection); W2 RAC GEMM; combine.
 * F % 32 == 0, H % 32 == 0.  The workspace holds every intermediate at the
 * offsets reported by moe_workspace_layout.  An expert index outside [0, E)
 * is invalid: its slot is computed as expert 0 but adds nothing to y, and
 * *status (device int32 [1], optional) is set to Q4_EINVAL. */
size_t moe_workspace_size(int32_t fmt, int64_t T, int32_t E, int32_t H, int32_t F,
                          int32_t topk, int32_t rac_k);
/* (host) offsets[0..Q4_MOE_WS_FIELDS-1] in bytes from the workspace base:
 *   0 perm int32 [T*topk]      1 offsets int32 [E+1]      2 x codes
 *   3 x scales                 4 x tensor scale fp32      5 x channel set int32 [rac_k]
 *   6 x residual R [T][kp]     7 h bf16 [T*topk][F]       8 h codes
 *   9 h scales                10 h tensor scale fp32     11 h channel set
 *  12 h residual R [T*topk][kp]     13 out [T*topk][H], Y's type (fp32 or bf16)
 *  14 x channel scores fp64 [H]                          15 h channel scores fp64 [F]
 * kp = rac_k rounded up to a multiple of 32.  R holds bf16(r) on the selected
 * channels (zero past rac_k), except for an NVFP4 GEMM that takes its
 * selected weight columns from a gathered copy (layers with more than 64
 * routed rows per expert on average, or K % 64 != 0): there it holds the fp16
 * operand bf16(r) 2^-e, s_t = f 2^e with f in [0.5, 1).  Decode-shaped layers
 * read the selected columns of W_hi^T inside the GEMM. */
#define Q4_MOE_WS_FIELDS 16
q4_status_t moe_workspace_layout(int32_t fmt, int64_t T, int32_t E, int32_t H, int32_t F,
                                 int32_t topk, int32_t rac_k, size_t *offsets);
q4_status_t moe_w4a4_grouped_gemm(int32_t fmt, const uint16_t *tokens, int64_t T, int32_t H,
                                  const int32_t *topk_idx, const float *topk_w, int32_t topk,
                                  int32_t E, int32_t F, const uint8_t *w13_codes,
                                  const uint8_t *w13_scales, const float *w13_tensor_scales,
                                  const uint8_t *w2_codes, const uint8_t *w2_scales,
                                  const float *w2_tensor_scales, const uint16_t *w13_hi_t,
                                  const uint16_t *w2_hi_t, const uint8_t *w13_scale_records,
                                  const uint8_t *w2_scale_records, const float *h_tensor_scale,
                                  int32_t rac_k, void *Y,
                                  int32_t y_dtype, void *workspace, size_t workspace_bytes,
                                  int32_t *status, void *stream);
/* moe_w4a4_grouped_gemm with option flags (the plain call is flags = 0):
 *   Q4_MOE_FUSE_H_QUANT  with h_tensor_scale (else Q4_EINVAL): where the W13
 *       GEMM can run on 256 x 256 tiles (prefill shapes: NVFP4, H % 128 == 0,
 *       2F % 256 == 0, H >= 1024, or H >= 512 with the weights' scale
 *       records), h is quantized in the W13 epilogue as it is produced: the
 *       fused stage of QUADS section 3.3 "Efficient implementation".  Codes,
 *       scales and the per-channel residual sums come out of the GEMM, with
 *       no separate pass over h.  Elsewhere the flag changes nothing.
 *       Results are those of the unfused call with the same h_tensor_scale,
 *       except that W13 then runs on 256 x 256 tiles rather than 128 x 512:
 *       h can differ from the unfused call's in the order of the sums of an
 *       expert's last rows, within the GEMM tolerance.  The epilogue's
 *       encoding runs beside no MFMA work, so the fused call can be slower
 *       than the unfused one.
 * Unknown flag bits: Q4_EINVAL. */
#define Q4_MOE_FUSE_H_QUANT 1u
q4_status_t moe_w4a4_grouped_gemm_ex(int32_t fmt, const uint16_t *tokens, int64_t T, int32_t H,
                                     const int32_t *topk_idx, const float *topk_w, int32_t topk,
                                     int32_t E, int32_t F, const uint8_t *w13_codes,
                                     const uint8_t *w13_scales, const float *w13_tensor_scales,
                                     const uint8_t *w2_codes, const uint8_t *w2_scales,
                                     const float *w2_tensor_scales, const uint16_t *w13_hi_t,
                                     const uint16_t *w2_hi_t, const uint8_t *w13_scale_records,
                                     const uint8_t *w2_scale_records, const float *h_tensor_scale,
                                     int32_t rac_k, void *Y,
                                     int32_t y_dtype, void *workspace, size_t workspace_bytes,
                                     int32_t *status, uint32_t flags, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* Q4RAC_H */
