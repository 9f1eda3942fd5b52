/*
 * qlin.h -- C ABI of libqlin, the outlier-aware quantized linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is assembled from three methods described on public pages:
 *   - "Quaff: Quantized Parameter-Efficient Fine-Tuning under Outlier Spatial
 *     Stability Hypothesis" (paper notes): INT8 weight-activation quantization,
 *     the decoupled form Y = X^(sW) = X^W + X^_{:,O}(s_O - 1)W_O with a sparse
 *     compensation term on a fixed outlier channel set O, and targeted momentum
 *     scaling s_t = gamma s_{t-1} + (1 - gamma) beta ("key design").
 *   - "QQQ: Quality Quattuor-Bit Quantization for Large Language Models"
 *     (review): W4A8 GEMMs, per-channel (INT4 -> INT8 by a left shift of 4,
 *     INT8 GEMM, INT32 -> FP16) and per-group (INT4 -> FP16, fused
 *     dequant-quant with the group/channel scale ratio, FP16 -> INT8, INT8
 *     GEMM, INT32 -> FP16) ("technical architecture", W4A8 GEMM kernels).
 *   - "OffQ: Taming Structured Outliers in LLM Quantization by Offsetting":
 *     a partially random Hadamard matrix with an all-ones first row turns the
 *     concentrated outlier channel of a group into a constant offset that the
 *     zero point of asymmetric quantization absorbs (methodology).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *     and allocates every buffer; the library keeps no pointer after return.
 *   - Tensors are row-major and contiguous.  fp16 values are passed as their
 *     uint16_t bit patterns.  X is [M x K] (tokens x input channels), W is
 *     [K x N] (input x output channels), Y is [M x N].
 *   - Every pointer must be 16-byte aligned (QLIN_ERR_ALIGN otherwise).
 *   - Shapes: M >= 0 (M == 0 returns QLIN_OK after the shape checks, reads no
 *     pointer and launches nothing, except qlin_momentum_update);
 *     K > 0 and K % 128 == 0; N > 0 and N % 64 == 0; every dimension below
 *     2^31 and every operand (M*K, K*N, M*N elements) at most 2^40, so that no
 *     size or index overflows 64 bits (QLIN_ERR_SHAPE otherwise).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream).  Nothing is synchronised; results are ready when the stream is.
 *   - Arguments are validated before any HIP call; a non-zero status means
 *     nothing was launched and no output was touched, except QLIN_ERR_HIP,
 *     which reports a failed launch.  qlin_last_error() gives a message.
 *   - No entry point allocates device memory or retains state between calls
 *     (qlin_momentum_update_noalloc aside: it works in a static device array,
 *     see there); calls on different streams touching disjoint outputs may
 *     overlap.
 *   - Rounding: every float -> integer decision is round-half-to-even in IEEE
 *     float32 (float16 where stated), one rounding per operation, no fused
 *     multiply-add, correctly rounded division and square root.
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qlin_status;
#define QLIN_OK 0
#define QLIN_ERR_INVALID_ARG 1 /* null pointer, negative size, bad enum value      */
#define QLIN_ERR_SHAPE 2       /* K % 128, N % 64, nO > K, sizes beyond the limits  */
#define QLIN_ERR_ALIGN 3       /* a pointer is not 16-byte aligned                  */
#define QLIN_ERR_UNSUPPORTED 4 /* a group size / bit width / block not provided     */
#define QLIN_ERR_HIP 5         /* the HIP runtime reported an error at launch       */

#define QLIN_ABI_VERSION 3

/* Weight layouts accepted by qlin_pack_weight / qlin_packed_bytes. */
#define QLIN_LAYOUT_W8 1  /* int8 codes for qlin_gemm_w8a8                         */
#define QLIN_LAYOUT_W4S 2 /* signed int4 codes [-8,7] for qlin_gemm_w4a8            */
#define QLIN_LAYOUT_W4U 3 /* unsigned int4 codes [0,15] for qlin_gemm_w4a4          */
#define QLIN_LAYOUT_WO 4  /* fp16 rows W_O [nO x N] for the compensation term       */
#define QLIN_LAYOUT_W8T 5 /* int8 codes [K x N] packed as their transpose [N x K]   */
                          /* (reduction over N) for qlin_quaff_backward; needs      */
                          /* N % 128 == 0 and K % 64 == 0                          */

/* Version of this ABI (QLIN_ABI_VERSION). Host only. */
int32_t qlin_abi_version(void);
/* Static name of a status code. Host only. */
const char* qlin_status_string(qlin_status status);
/* Message describing the last non-zero status returned on this host thread. */
const char* qlin_last_error(void);
/* Row stride of the per-outlier arrays qO / xO: nO rounded up to a multiple of 16. Host only. */
int32_t qlin_outlier_ld(int32_t nO);

/* ------------------------------------------------------------------------
 * Activation side
 * --------------------------------------------------------------------- */

/*
 * qlin_quant_act -- per-token symmetric int8 quantization, optionally of X*r.
 * Quaff notes, "key design" (INT8 activations; with momentum scaling the
 * quantized operand is X^ = Q(X / s), here X times r = 1/s) and QQQ review,
 * "technical architecture" (8-bit per-token activations).
 *   x      fp16 [M x K]
 *   r      fp32 [K] per-channel multiplier, or NULL for none
 *   q      int8 [M x K] out: clamp(rint(v * inv), -127, 127) with v = x * r,
 *          a = max_k |v|, inv = 127 / a (0 if a == 0)
 *   scale  fp32 [M] out: a / 127 (0 if a == 0)
 * Outlier columns (for the Quaff compensation term), written with the row
 * stride ldO = qlin_outlier_ld(nO), columns nO..ldO-1 zero:
 *   O, nO  int32 [nO] channel indices (an index outside [0, K) gives 0)
 *   qO     int8 [M x ldO] out or NULL: q[:, O]
 *   xO     fp16 [M x ldO] out or NULL: fp16(q[:, O] * (s[O] - 1)), the operand
 *          X^_{:,O}(s_O - 1) of the compensation term without the token step
 *   s      fp32 [K] (required with xO)
 * With nO == 0, O, qO and xO must be NULL; with nO > 0, qO or xO is required.
 */
qlin_status qlin_quant_act(const uint16_t* x, int64_t M, int64_t K, const float* r,
                           int8_t* q, float* scale, const int32_t* O, int32_t nO, const float* s,
                           int8_t* qO, uint16_t* xO, void* stream);

/*
 * qlin_hadamard_offset -- OffQ activation path (OffQ, methodology,
 * "absorption via offsetting").  Per token and per group of `block` channels:
 * t = (x * d) H_block, with H the natural-order Sylvester matrix (row 0 all
 * ones), evaluated exactly and rounded once to fp32.  Then per token:
 * rng = max t - min t, inv = 15 / rng, step = rng / 15 (both 1 if rng == 0),
 * z = rint(-min t * inv), code = clamp(rint(t * inv) + z, 0, 15).
 *   x       fp16 [M x K]
 *   signs   int8 [K]: a negative entry means -1, any other +1; OffQ's all-ones
 *           first row needs signs[block*b] == +1 (not checked)
 *   block   128 (the only size provided)
 *   q4      uint8 [M x K/2] out: two codes per byte, low nibble = even k
 *   scale   fp32 [M] out: step
 *   zero    int32 [M] out: z
 *   rowsum  int32 [M] out: sum_k code (used by the W4A4 zero-point epilogue)
 *   t       fp32 [M x K] out, or NULL: the transformed values (for checking)
 */
qlin_status qlin_hadamard_offset(const uint16_t* x, int64_t M, int64_t K, const int8_t* signs,
                                 int32_t block, uint8_t* q4, float* scale, int32_t* zero,
                                 int32_t* rowsum, float* t, void* stream);

/*
 * qlin_hadamard_offset_group -- OffQ's group-wise offsets (OffQ, methodology,
 * "grouped implementation": each group of channels gets its own scale and
 * zero point, which absorb that group's outlier; the ablations settle on
 * groups of 128).  The transform of qlin_hadamard_offset, then the same
 * asymmetric rule applied to every group g of `block` channels of a token
 * separately (range of the group's own values).  G = K / block.
 *   x, signs, block, q4, t  as in qlin_hadamard_offset
 *   scale   fp32 [M x G] out: step of group g of token m at m * G + g
 *   zero    int32 [M x G] out: z
 *   rowsum  int32 [M x G] out: sum of the group's codes
 */
qlin_status qlin_hadamard_offset_group(const uint16_t* x, int64_t M, int64_t K, const int8_t* signs,
                                       int32_t block, uint8_t* q4, float* scale, int32_t* zero,
                                       int32_t* rowsum, float* t, void* stream);

/*
 * qlin_momentum_update -- Quaff targeted momentum scaling, one step
 * (Quaff notes, "key design"): for o in O, c = max_m |x[m,o]|,
 * beta = max(1, sqrt(c / wmax_O[o])) (beta = 1 if wmax_O[o] == 0 or M == 0),
 * s[o] = (gamma * s[o]) + ((1 - gamma) * beta); then r[k] = 1 / s[k] for all k.
 * Channels outside O keep their s (the caller starts from s = 1).  M may be 0
 * (then beta = 1 for every o).
 *   x       fp16 [M x K] the current batch (unscaled)
 *   O, nO   int32 [nO], strictly increasing (not checked on the host: entries
 *           outside [0, K) are skipped, and a decreasing or repeated entry
 *           leaves s and r unspecified but in bounds); nO may be 0
 *   wmax_O  fp32 [nO]: max_n |W[O[j], n]| (qlin_weight_row_absmax)
 *   gamma   momentum in [0, 1]
 *   s       fp32 [K] in/out;  r fp32 [K] out
 *   work    device workspace of qlin_momentum_work_bytes(M, nO) bytes, or
 *           NULL.  With a workspace and M >= 4096 the column maxima are taken
 *           by up to 16 row blocks per 64-channel strip in one launch and
 *           folded per outlier channel in a second (every CU reads part of
 *           x); otherwise one launch with one workgroup per strip.  Same
 *           result either way.  The workspace holds partial maxima until the
 *           call's kernels end; calls that overlap must not share it.
 */
qlin_status qlin_momentum_update(const uint16_t* x, int64_t M, int64_t K, const int32_t* O,
                                 int32_t nO, const float* wmax_O, float gamma, float* s, float* r,
                                 float* work, void* stream);

/* Bytes of the qlin_momentum_update workspace for M tokens and nO outliers
 * (0 for negative arguments). Host only. */
size_t qlin_momentum_work_bytes(int64_t M, int32_t nO);

/*
 * qlin_quaff_momentum_quant -- one Quaff step's activation side in one call:
 * the momentum update of qlin_momentum_update, then qlin_quant_act of x with
 * the new r and the compensation operand xO with the new s (Quaff notes,
 * "key design": targeted momentum scaling, then the INT8 quantization of the
 * decoupled form).  Bit-identical to those two calls in that order.
 *   x, M, K, O, nO, wmax_O, gamma, s, r   as in qlin_momentum_update
 *   work    device workspace of qlin_quaff_momentum_quant_work_bytes(M, nO)
 *           bytes, or NULL.  With it (and 1 <= nO <= 256, K <= 8192) the
 *           maxima are taken by every CU over 4 row blocks per 64-channel
 *           strip, and each quantizer lane folds them for its outlier
 *           slots into the new s[O], r[O] (two launches in all, none for
 *           the fold); otherwise the two calls above are made.  Calls that
 *           overlap must not share it.  Between the two launches r holds a
 *           marker (a NaN) at each outlier channel; s must hold finite
 *           positive values, as the momentum update keeps them.
 *   q, scale, xO   as in qlin_quant_act (xO required when nO > 0, NULL
 *           otherwise; qO, the outlier columns' codes alone, is not offered)
 * M == 0 runs the momentum update alone.
 */
qlin_status qlin_quaff_momentum_quant(const uint16_t* x, int64_t M, int64_t K, const int32_t* O,
                                      int32_t nO, const float* wmax_O, float gamma, float* s,
                                      float* r, float* work, int8_t* q, float* scale, uint16_t* xO,
                                      void* stream);

/* Bytes of the qlin_quaff_momentum_quant workspace for M tokens and nO
 * outliers (0 for negative arguments). */
size_t qlin_quaff_momentum_quant_work_bytes(int64_t M, int32_t nO);

/*
 * qlin_momentum_update_noalloc -- qlin_momentum_update without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, result and rounding as
 * qlin_momentum_update with a workspace; the partial maxima live in a static
 * device array of the library, one per GPU, held until the process ends
 * (16 row blocks x 8192 outlier channels of fp32, 512 KiB).
 *   nO      at most 8192 (QLIN_ERR_SHAPE otherwise, before any HIP call)
 * The first call on a device looks up the array's address on that device
 * (the device of `stream`).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * host threads) race and give undefined s and r; calls in one stream are
 * ordered and do not.  No part of the array needs to start at zero.
 */
qlin_status qlin_momentum_update_noalloc(const uint16_t* x, int64_t M, int64_t K, const int32_t* O,
                                         int32_t nO, const float* wmax_O, float gamma, float* s,
                                         float* r, void* stream);

/* ------------------------------------------------------------------------
 * Weight preparation (offline; W is frozen)
 * --------------------------------------------------------------------- */

/*
 * qlin_quant_weight_sym -- symmetric per-output-channel weights (QQQ review,
 * "technical architecture", per-channel W4A8; Quaff notes, "overall
 * framework", W_int).  a_n = max_k |W[k,n]|, step_n = fp16(a_n / qmax),
 * code = clamp(rint(W / step_n), lo, qmax); (qmax, lo) = (127, -127) for
 * bits = 8 and (7, -8) for bits = 4; a zero step gives zero codes.
 *   w      fp16 [K x N];  codes int8 [K x N] out;  scale fp16 [N] out
 */
qlin_status qlin_quant_weight_sym(const uint16_t* w, int64_t K, int64_t N, int32_t bits,
                                  int8_t* codes, uint16_t* scale, void* stream);

/*
 * qlin_quant_weight_group -- QQQ per-group int4 weights with the folded
 * requantization ratio (QQQ review, "technical architecture", per-group W4A8
 * GEMM and FusedDequantQuant).  s_g = fp16(max_{k in g}|W| / 7),
 * code = clamp(rint(W / s_g), -8, 7), s_c = fp16(max_k |W| / 127),
 * ratio = fp16(s_g / s_c) (0 where s_c == 0).
 *   group   128 (the only size provided)
 *   codes   int8 [K x N] out;  group_scale fp16 [K/group x N] out;
 *   channel_scale fp16 [N] out;  ratio fp16 [K/group x N] out
 */
qlin_status qlin_quant_weight_group(const uint16_t* w, int64_t K, int64_t N, int32_t group,
                                    int8_t* codes, uint16_t* group_scale,
                                    uint16_t* channel_scale, uint16_t* ratio, void* stream);

/*
 * qlin_quant_weight_offq -- OffQ weight side: W'' = blockdiag(H'^-1) W with
 * H' = diag(signs) H_block and H'^-1 = H_block diag(signs) / block, exact,
 * rounded once to fp32; then per output channel the asymmetric int4 rule of
 * qlin_hadamard_offset over k.  (x H')(H'^-1 W) = x W, so the layer output is
 * preserved (OffQ, methodology).
 *   codes  uint8 [K x N] out (0..15, one per byte);  scale fp32 [N];
 *   zero int32 [N];  colsum int32 [N] (sum_k code)
 */
qlin_status qlin_quant_weight_offq(const uint16_t* w, int64_t K, int64_t N, const int8_t* signs,
                                   int32_t block, uint8_t* codes, float* scale, int32_t* zero,
                                   int32_t* colsum, void* stream);

/*
 * qlin_weight_row_absmax -- out[i] = max_n |w_rows[i, n]| (fp32), the max|W_i|
 * of Quaff's beta for the rows W_O (Quaff notes, "key design").
 *   w_rows fp16 [R x N] (R >= 0);  out fp32 [R]
 */
qlin_status qlin_weight_row_absmax(const uint16_t* w_rows, int64_t R, int64_t N, float* out,
                                   void* stream);

/*
 * qlin_weight_colsum_group -- column sums of weight codes over each group of
 * `group` k, for the group-wise W4A4 zero-point correction (OffQ, methodology,
 * "grouped implementation": the activation zero point changes per group).
 *   codes    uint8 [K x N] (one code per byte, as from qlin_quant_weight_offq)
 *   group    128 (the only size provided)
 *   colsum_g int32 [K/group x N] out: colsum_g[g, n] = sum_{k in group g} codes[k, n]
 */
qlin_status qlin_weight_colsum_group(const uint8_t* codes, int64_t K, int64_t N, int32_t group,
                                     int32_t* colsum_g, void* stream);

/* ------------------------------------------------------------------------
 * OffQ concentration, Top-1 PCA (offline calibration; OffQ, methodology,
 * "concentration via Top-1 PCA": only the most extreme token of each
 * calibration sequence enters the covariance; its leading eigenvector is
 * rotated into the first channel, and the weights take the inverse rotation)
 * --------------------------------------------------------------------- */

/*
 * qlin_pca_select -- per sequence s, the token t = argmax_t max_k |x[s,t,k]|
 * (fp32 of the fp16 values; the first such t on ties) and a copy of it.
 *   x    fp16 [S x T x K], K % 8 == 0;  idx int32 [S] out;  z fp16 [S x K] out
 */
qlin_status qlin_pca_select(const uint16_t* x, int64_t S, int64_t T, int64_t K, int32_t* idx, uint16_t* z,
                            void* stream);

/*
 * qlin_pca_leading_eigvec -- leading eigenvector v (unit, v[0] <= 0) and its
 * eigenvalue of the sample covariance C = Zc^T Zc / (S - 1) of the rows of z,
 * centred on their mean, by power iteration in float64 without forming C
 * (the iterates are kept as token weights a, v = Zc^T a, through the S x S
 * Gram matrix Zc Zc^T).  The start vector is the centred row of largest
 * norm; the iteration stops when successive vectors differ by less than tol
 * (2-norm) or after max_iter.
 *   z fp16 [S x K] (2 <= S <= 2048, K % 8 == 0, K <= 8192);  v float64 [K] out;
 *   lambda float64 [1] out;  iters int32 [1] out (iterations run);
 *   ws float64 scratch [S*S + K + S + 1]
 * A calibration step, not a per-token one.
 */
qlin_status qlin_pca_leading_eigvec(const uint16_t* z, int64_t S, int64_t K, int32_t max_iter, double tol,
                                    double* v, double* lambda, int32_t* iters, double* ws, void* stream);

/*
 * qlin_pca_fold_weight -- w_out = fp16(H W) with the Householder reflection
 * H = I - beta u u^T, u = v - e_0, beta = 2 / (u^T u), so H v = e_0 and
 * (x H)(H W) = x W (H is its own inverse).  float64 arithmetic, one rounding.
 *   w fp16 [K x N] (K <= 65535, N % 8 == 0);  v float64 [K] (unit, v[0] <= 0);
 *   w_out fp16 [K x N] out (may not alias w; also holds partial sums until
 *   the last pass);  ws float64 scratch [N]
 */
qlin_status qlin_pca_fold_weight(const uint16_t* w, int64_t K, int64_t N, const double* v, uint16_t* w_out,
                                 double* ws, void* stream);

/*
 * qlin_pca_rotate -- x_out = fp16(x H) for tokens x [M x K] (the activation
 * side of the same rotation: x - beta (x . u) u^T in float64, one rounding).
 * K % 8 == 0 and K <= 8192.  Where a preceding layer can absorb H offline,
 * this kernel is not needed.
 */
qlin_status qlin_pca_rotate(const uint16_t* x, int64_t M, int64_t K, const double* v, uint16_t* x_out,
                            void* stream);

/* Bytes of a packed weight buffer for `layout` (0 for invalid arguments). Host only. */
size_t qlin_packed_bytes(int32_t layout, int64_t K, int64_t N);

/*
 * qlin_pack_weight -- reorder one-code-per-byte weights [K x N] into the
 * tiled layout the GEMMs read (int4 layouts hold two codes per byte, eight per
 * 32-bit word).  The layout is private to the library: only pass the result to
 * the matching GEMM.  codes: int8 [K x N] for W8 / W4S, uint8 for W4U, fp16
 * [nO x N] for WO (then K = nO, any positive value, rows padded to
 * qlin_outlier_ld(nO) with zeros).
 *   packed: qlin_packed_bytes(layout, K, N) bytes out.
 */
qlin_status qlin_pack_weight(int32_t layout, const void* codes, int64_t K, int64_t N, void* packed,
                             void* stream);

/* ------------------------------------------------------------------------
 * GEMMs with fused epilogues
 * --------------------------------------------------------------------- */

/*
 * qlin_gemm_w8a8 -- int8 x int8 -> int32, fused dequant, optional fused Quaff
 * compensation (Quaff notes, "key design", decoupled WAQ).
 *   acc[m,n] = sum_k qa[m,k] * W8[k,n]
 *   y[m,n]   = fp16(sa[m] * (acc[m,n] * sw[n] + sum_j xO[m,j] * WO[j,n]))
 * The second term is the sparse X^_{:,O}(s_O - 1)W_O with
 * X^_{m,o} = q[m,o] * sa[m] and xO = fp16(q[:, O] * (s[O] - 1)) from
 * qlin_quant_act; it is skipped when nO == 0 (then xO and WO must be NULL).
 * fp32 accumulation of fp16 products.
 *   qa  int8 [M x K];  sa fp32 [M];  w8 packed QLIN_LAYOUT_W8;  sw fp16 [N]
 *   xO  fp16 [M x qlin_outlier_ld(nO)];  WO packed QLIN_LAYOUT_WO (nO rows)
 *   y   fp16 [M x N] out;  acc int32 [M x N] out or NULL
 */
qlin_status qlin_gemm_w8a8(const int8_t* qa, const float* sa, const void* w8, const uint16_t* sw,
                           int64_t M, int64_t N, int64_t K, const uint16_t* xO, int32_t nO,
                           const void* WO, uint16_t* y, int32_t* acc, void* stream);

/*
 * qlin_gemm_w4a8 -- QQQ W4A8 (QQQ review, "technical architecture").
 * group == 0, per channel: each int4 weight is moved to the high half of a
 * byte (a left shift by 4, i.e. 16 * q4 as int8), multiplied in int8, and the
 * sum is divided by 16 exactly: acc = sum_k qa * q4;  y = fp16(acc * sa * sw).
 * group == 128, per group: w8 = clamp(rint(fp16(q4 * ratio[k/128, n])), -127, 127)
 * (one fp16 rounding of the exact product, then round half to even);
 * acc = sum_k qa * w8;  y = fp16(acc * sa * sw) with sw = s_c.  The
 * requantization runs inside the K loop of every tile, or, given a
 * workspace and more than 128 tokens, once per call into `work` (the int8
 * weights in QLIN_LAYOUT_W8 order), after which the int8 tile reads them from
 * there: the same acc and y bit for bit, with the vector work done once
 * instead of once per 128- or 256-row tile.
 *   qa int8 [M x K];  sa fp32 [M];  w4 packed QLIN_LAYOUT_W4S;  sw fp16 [N]
 *   ratio fp16 [K/128 x N] (group == 128) or NULL (group == 0)
 *   y fp16 [M x N] out;  acc int32 [M x N] out or NULL
 *   work  device scratch of qlin_gemm_w4a8_work_bytes(M, N, K, group) bytes,
 *         16-byte aligned, overlapping no other argument, or NULL; its
 *         contents on entry do not matter and are left undefined.  Ignored
 *         when that size is 0 (per channel, or M <= 128).  Calls that share
 *         a workspace must be ordered (one stream).
 */
qlin_status qlin_gemm_w4a8(const int8_t* qa, const float* sa, const void* w4, const uint16_t* sw,
                           const uint16_t* ratio, int32_t group, int64_t M, int64_t N, int64_t K,
                           uint16_t* y, int32_t* acc, void* work, void* stream);
/* Workspace bytes qlin_gemm_w4a8 uses for these arguments: K * N for
 * group == 128 with M > 128 and valid shapes, else 0. Host only. */
size_t qlin_gemm_w4a8_work_bytes(int64_t M, int64_t N, int64_t K, int32_t group);

/*
 * qlin_gemm_w4a4 -- asymmetric int4 x int4 on int8 matrix cores with the
 * zero-point correction in the epilogue (OffQ: uniform 4-bit weights and
 * activations with zero points, methodology and "core contributions").
 *   raw = sum_k qa * qw (codes 0..15)
 *   acc = raw - zw[n]*rowsum[m] - za[m]*colsum[n] + K*za[m]*zw[n]
 *       = sum_k (qa - za[m]) (qw - zw[n])           (int32)
 *   y   = fp16(acc * sa[m] * sw[n])
 * Precondition: the true sum fits int32, |sum_k (qa - za)(qw - zw)| < 2^31;
 * K * (|za| + 15) * (|zw| + 15) < 2^31 is sufficient.  The expansion is
 * evaluated in wrapping 32-bit arithmetic, so its intermediate terms may
 * exceed int32 without harm; a true sum outside int32 wraps silently (not
 * checked on the device).
 *   qa4 uint8 [M x K/2] (low nibble = even k), sa fp32 [M], za int32 [M],
 *   rowsum int32 [M];  w4 packed QLIN_LAYOUT_W4U;  sw fp32 [N], zw int32 [N],
 *   colsum int32 [N];  y fp16 [M x N] out;  acc int32 [M x N] out or NULL
 */
qlin_status qlin_gemm_w4a4(const uint8_t* qa4, const float* sa, const int32_t* za,
                           const int32_t* rowsum, const void* w4, const float* sw,
                           const int32_t* zw, const int32_t* colsum, int64_t M, int64_t N,
                           int64_t K, uint16_t* y, int32_t* acc, void* stream);

/*
 * qlin_gemm_w4a4_group -- W4A4 with OffQ's group-wise activation offsets
 * (OffQ, methodology, "grouped implementation"): a step sa, zero point za and
 * code sum per token and group of 128 k (from qlin_hadamard_offset_group),
 * per-channel asymmetric int4 weights.  With G = K / 128:
 *   raw_g = sum_{k in g} qa * qw                                  (int32, exact)
 *   acc_g = sum_{k in g} (qa - za[m,g]) (qw - zw[n])
 *         = raw_g - za[m,g] * colsum_g[g,n] - zw[n] * (rowsum[m,g] - 128 za[m,g])
 *   y     = fp16(sw[n] * sum_g sa[m,g] * acc_g)
 * Evaluation in fp32, per element:
 *   Z = sum_g w_g[m] * colsum_g[g,n],  w_g = -fp32(sa[m,g] * za[m,g]),
 *   then F = Z and, group by group in g order, F = fma(sa[m,g], fp32(raw_g), F);
 *   per token P = sum_g fma(sa[m,g], fp32(rowsum[m,g] - 128 za[m,g]), .);
 *   y = fp16((F - zw[n] * P) * sw[n]).
 * Z runs on fp16 matrix cores with fp32 accumulation: colsum_g <= 1920 is
 * exact in fp16; per token and chunk of 32 groups, w is scaled by the power of
 * two that puts the chunk's largest |w| in [2^14, 2^15) and split into fp16
 * hi + lo halves, which carry each w to within 2^-21 of that largest |w|
 * (relative to max|sa * za| of the chunk), before the fp32 sums are scaled
 * back exactly.  The fp16 output therefore lies within the normwise 1e-3 of
 * the exact value whenever the terms do not cancel far below
 * max|sa * za| * colsum; precondition |za| < 2^12 (not checked on the device).
 *   qa4 uint8 [M x K/2] (low nibble = even k);  sa fp32 [M x G];
 *   za int32 [M x G];  rowsum int32 [M x G];  w4 packed QLIN_LAYOUT_W4U;
 *   sw fp32 [N];  zw int32 [N];  colsum_g int32 [G x N] (qlin_weight_colsum_group;
 *   16-byte aligned);  y fp16 [M x N] out;
 *   acc int32 [G x M x N] out or NULL: raw_g[g, m, n] at (g * M + m) * N + n,
 *   the exact integer sums the fp32 evaluation starts from (for checking;
 *   writing them makes the call slower).
 */
qlin_status qlin_gemm_w4a4_group(const uint8_t* qa4, const float* sa, const int32_t* za,
                                 const int32_t* rowsum, const void* w4, const float* sw,
                                 const int32_t* zw, const int32_t* colsum_g, int64_t M, int64_t N,
                                 int64_t K, uint16_t* y, int32_t* acc, void* stream);

/*
 * qlin_quaff_backward -- input gradient of the Quaff layer under the
 * straight-through estimator (Quaff notes, "loss function / training
 * strategy": standard STE; the forward is the decoupled form of "key design").
 * STE passes the gradient through the quantizer, so with W-hat = W_int * sw:
 *   dX = (dY W-hat^T + scatter_O(dY W_O^T * (s_O - 1))) * r
 * The main product runs on int8 matrix cores: the weight step sw[n] lies along
 * its reduction, so it moves to the gradient, G = dY * sw (fp32), which is
 * quantized per token like the forward activations (gq, gs: the rule of
 * qlin_quant_act).  Then
 *   acc[m,k] = sum_n gq[m,n] * W_int[k,n]                     (int32)
 *   cb[m,j]  = sum_n dY[m,n] * W_O[j,n]                        (fp32, fp16 products)
 *   dX[m,k]  = fp16(r[k] * (gs[m] * acc[m,k] + [k = O[j]] (s[k] - 1) * cb[m,j]))
 * Three launches on `stream`.  The caller provides the intermediates.
 *   dy   fp16 [M x N];  sw fp16 [N] (the forward weight steps)
 *   w8t  W_int packed with QLIN_LAYOUT_W8T (K x N codes; N % 128 == 0)
 *   s, r fp32 [K]: the momentum state of the forward step (r = 1 / s)
 *   O, nO  int32 [nO], strictly increasing;  w_o fp16 [nO x N] row-major: the
 *          rows W_O (not packed).  With nO == 0, O, w_o and cb must be NULL.
 *   gq int8 [M x N], gs fp32 [M], cb fp32 [M x qlin_outlier_ld(nO)]: scratch
 *          written here (gq, gs: the quantized gradient; cb as above, zero in
 *          the columns nO..ldO-1)
 *   dx fp16 [M x K] out;  acc int32 [M x K] out or NULL
 */
qlin_status qlin_quaff_backward(const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint16_t* sw,
                                const void* w8t, const float* s, const float* r, const int32_t* O, int32_t nO,
                                const uint16_t* w_o, int8_t* gq, float* gs, float* cb, uint16_t* dx,
                                int32_t* acc, void* stream);

/*
 * qlin_outlier_comp -- the sparse compensation term on its own, added to an
 * existing output (Quaff notes, "key design"):
 *   y[m,n] = fp16(y[m,n] + sa[m] * sum_j xO[m,j] * WO[j,n])
 *   xO fp16 [M x qlin_outlier_ld(nO)] (from qlin_quant_act);  sa fp32 [M];
 *   WO packed QLIN_LAYOUT_WO;  y fp16 [M x N] in/out.  nO == 0 leaves y unchanged.
 */
qlin_status qlin_outlier_comp(const uint16_t* xO, const float* sa, int32_t nO, const void* WO,
                              int64_t M, int64_t N, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
