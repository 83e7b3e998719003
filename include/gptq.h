/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library.
 *
 * One linear layer W (d_out x d_in, row-major, column j = input channel j) is
 * quantized from calibration activations X (tokens x d_in, token-major) in
 * four stream-ordered calls:
 *
 *   gptq_hessian_accumulate   S += X^T X (fp32, lower triangle), D += diag in fp64
 *   gptq_prepare_hinv         H = 2 S / N, damping, optional importance order,
 *                             U = upper Cholesky factor of the damped inverse
 *   gptq_quantize_layer       column-by-column group quantization with error
 *                             feedback through the rows of U
 *   gptq_pack_int4 / gptq_pack_bits   dense packing of the integer codes
 *
 * The method is the one the pages "3. 模型量化技术(下)" (section GPTQ：基于二阶
 * 信息的后训练量化, pseudocode block), "INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍"
 * (sections 一 and 三) and ipipp.com's "GPTQ：在每一列权重上做二阶误差补偿"
 * (quantize_gptq listing and the paragraph before it) describe.
 *
 * Conventions shared by every call:
 *   - Every buffer is owned and allocated by the caller; the library never
 *     allocates or frees device memory.  Scratch memory is a caller-provided
 *     device "workspace" whose size gptq_workspace_size() reports.
 *   - Device pointers are addresses in the current HIP device's memory;
 *     "host" pointers are ordinary process memory read synchronously.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Each call checks
 *     its arguments synchronously (returning GPTQ_EINVAL / GPTQ_EUNSUPPORTED
 *     before touching the GPU), then enqueues kernels on `stream` and returns;
 *     results are valid once the stream has been synchronized.
 *   - A HIP launch or runtime failure returns GPTQ_EHIP.
 *   - Calls on distinct streams with distinct buffers may run concurrently
 *     from several threads.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPTQ_ABI_VERSION 5

typedef enum {
  GPTQ_OK = 0,
  GPTQ_EINVAL = 1,        /* bad argument (null pointer, size, layout) */
  GPTQ_ENOTPD = 2,        /* reserved for bindings: info != 0 after prepare */
  GPTQ_EHIP = 3,          /* HIP runtime or launch failure */
  GPTQ_EUNSUPPORTED = 4,  /* valid request this build does not implement */
  GPTQ_ENOMEM = 5         /* workspace smaller than gptq_workspace_size() */
} gptq_status;

typedef enum { GPTQ_F32 = 0, GPTQ_F16 = 1, GPTQ_BF16 = 2 } gptq_dtype;

typedef enum {
  GPTQ_OP_HESSIAN = 0,
  GPTQ_OP_PREPARE = 1,
  GPTQ_OP_QUANTIZE = 2,
  GPTQ_OP_W4A16 = 3,
  GPTQ_OP_ABS = 4,
  GPTQ_OP_AWQ_SEARCH = 5,
  GPTQ_OP_FORWARD = 6
} gptq_op;

/* Quantizer and schedule parameters.
 *   bits        code width, 2..8 (4 = INT4; 3 = INT3).  maxq = 2^bits - 1.
 *   group_size  g: consecutive columns (in quantization order) that share one
 *               fp16 scale and one integer zero ("INT4/INT8 量化推理", section
 *               一: every 128 consecutive weights share a scale and a zero).
 *               Must divide d_in and be 16, 32, 64 or a multiple of 128
 *               (other divisors of 128 down to 4 pass validation but return
 *               GPTQ_EUNSUPPORTED).
 *   block_size  columns whose error feedback is applied inside one tile before
 *               the deferred ("lazy") update of the later columns (ipipp.com
 *               page, section 一: process in blocks).  Must be 128.
 *   damp_rel    lambda = damp_rel * mean(diag H), added to the diagonal.
 *   act_order   nonzero: quantize columns in descending diag(H) order (same
 *               page: order the columns by importance), ties to the lower
 *               index.
 *   sym         0: asymmetric min-max groups (scale from the range, integer
 *               zero from the minimum).  1: symmetric groups (ipipp.com
 *               page, section 一, GPTQ listing and the remark after it: scale
 *               from the largest magnitude over 2^(bits-1) - 1, signed code
 *               clamped to [-2^(bits-1), 2^(bits-1) - 1], per group as real
 *               frameworks do): the zero is the fixed 2^(bits-1) and the
 *               stored code is the signed code plus that zero.  Other values
 *               are GPTQ_EINVAL.
 *   static_groups  0: a group's scale and zero come from its current values
 *               when its first column (in quantization order) is reached.
 *               1: every group's scale and zero are fixed before the column
 *               loop from W as given, over g consecutive ORIGINAL columns;
 *               with act_order a column is quantized in permuted order with
 *               its original group's parameters (the pages do not describe
 *               this option; it keeps g_idx[c] = c / g).  Other values are
 *               GPTQ_EINVAL. */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int32_t block_size;
  float damp_rel;
  int32_t act_order;
  int32_t sym;
  int32_t static_groups;
} gptq_params;

int32_t gptq_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* gptq_status_string(int32_t status);

/* Workspace bytes one call of `op` needs for the given shapes.
 *   GPTQ_OP_HESSIAN:  d_in, n_rows = rows of X handed to one call (the total
 *                     over all batch entries when row_idx is used), batch.
 *   GPTQ_OP_PREPARE:  d_in, batch.
 *   GPTQ_OP_QUANTIZE: p, d_out, d_in, batch.
 *   GPTQ_OP_W4A16:    d_out, d_in, n_rows = M (tokens of one call).
 *   GPTQ_OP_ABS:      d_in, n_rows (as GPTQ_OP_HESSIAN).
 *   GPTQ_OP_AWQ_SEARCH: d_out, d_in, n_rows = sample tokens n_s,
 *                     batch = number of candidate alphas.
 *   GPTQ_OP_FORWARD:  d_out, d_in, n_rows = tokens of one call.
 * Unused arguments are ignored (p may be NULL except for GPTQ_OP_QUANTIZE).
 * Writes *bytes_out (host). */
gptq_status gptq_workspace_size(int32_t op, const gptq_params* p, int64_t d_out, int64_t d_in,
                                int64_t n_rows, int64_t batch, size_t* bytes_out);

/* Hessian accumulation, H = 2 X^T X / N ("3. 模型量化技术(下)" pseudocode:
 * H from the layer's calibration inputs; ipipp.com listing: 2 (X^T X) / N).
 * The running state is (S, D, n_tokens), all in device memory; zero them
 * before the first call, then call once per chunk of calibration rows.  The
 * count stays on the device, so a call never waits for the GPU.
 *
 *   S         device fp32 [batch][d_in][d_in].  S[i][j] += sum_t X[t][i] X[t][j]
 *             for i >= j only; entries with i < j are neither read nor written.
 *             bf16/fp16 products are exact in fp32 and accumulate in fp32.
 *   D         device fp64 [batch][d_in].  D[i] += sum_t X[t][i]^2 in fp64 (the
 *             importance key and the damping mean use D).
 *   n_tokens  device int64 [batch]; += number of rows that entry used: all
 *             n_rows rows of X for a dense call, the indices inside
 *             [0, n_rows) for a gathered one (H = 2 S / N is then the mean
 *             over the rows that really contributed).
 *   X         device, n_rows x d_in elements of x_dtype, row stride ld_x
 *             elements; 16-byte aligned, ld_x * sizeof(elem) % 16 == 0,
 *             d_in % 8 == 0.
 *   row_idx   optional device int32 list of rows of X (gather, e.g. the tokens
 *             routed to each expert of an MoE layer); NULL = every row of X
 *             for a single entry (batch must be 1).  An index outside
 *             [0, n_rows) is skipped: never dereferenced, adds nothing to S,
 *             D or n_tokens.
 *   row_ptr   host int64 [batch + 1] when row_idx is given: entry b uses
 *             row_idx[row_ptr[b] .. row_ptr[b+1]).  Ignored otherwise.
 *   workspace device scratch of ws_bytes (see gptq_workspace_size).
 * The result is deterministic: no floating-point atomics; partial sums are
 * reduced in a fixed order. */
gptq_status gptq_hessian_accumulate(float* S, double* D, int64_t* n_tokens, const void* X,
                                    int32_t x_dtype, int64_t n_rows, int64_t d_in, int64_t ld_x,
                                    const int32_t* row_idx, const int64_t* row_ptr,
                                    int64_t batch, void* workspace, size_t ws_bytes, void* stream);

/* Damping, importance order and the inverse-Hessian factor (ipipp.com page,
 * section 一: damping H + eps I, inverse of H, optional importance order;
 * "INT4/INT8 量化推理", section 三: feedback through rows of H^-1).
 *
 *   H0 = 2 S / N (diagonal 2 D / N), lambda = damp_rel * mean(2 D / N),
 *   Hd = H0 + lambda I.  If act_order, perm = stable argsort of -D, else the
 *   identity.  U (upper triangular) satisfies U^T U = (Hd[perm][:, perm])^-1;
 *   row k of U scaled by U[k][k] is row k of the inverse of the sub-Hessian of
 *   the columns not yet quantized when column k is reached, which is the
 *   exact form of the pages' update.  Computed in fp64 (Cholesky of the
 *   reversed Hd, then its triangular inverse), stored as fp32.
 *
 *   S, D      device, as produced by gptq_hessian_accumulate (unchanged here).
 *   n_tokens  device int64 [batch] (the Hessian state's count).  An entry
 *             with N = 0 gets info = -1.
 *   U         device fp32 [batch][d_in][d_in]; entries below the diagonal are 0.
 *   perm      device int32 [batch][d_in]: perm[k] = original column quantized
 *             k-th.  May be NULL when act_order == 0.
 *   info      device int32 [batch]: 0 on success; -1 if the entry has no
 *             calibration rows (N = 0); k + 1 if Hd is not positive
 *             definite, k being the position (in quantization order) of the
 *             failing pivot -- the factorization runs from the last position
 *             backwards, so k is the largest such position.  U is then not
 *             meaningful.
 * For d_in >= 2048 part of the fp64 products runs on a second stream that the
 * library keeps per device (default priority); it starts after the work
 * enqueued on `stream` before this call and the work enqueued on `stream`
 * after it waits for it, so the call stays ordered like a single-stream
 * launch.  Calls from several host threads take turns at enqueueing. */
gptq_status gptq_prepare_hinv(const float* S, const double* D, const int64_t* n_tokens,
                              int64_t d_in, int64_t batch, const gptq_params* p, float* U,
                              int32_t* perm, int32_t* info, void* workspace, size_t ws_bytes,
                              void* stream);

/* Column-by-column quantization with error feedback ("INT4/INT8 量化推理",
 * section 三 listing; ipipp.com quantize_gptq listing), in blocks of 128
 * columns with a deferred update of the later columns.
 *
 * For column k (quantization order): at a group start the group's scale and
 * zero come from its current values: xmin = min(0, min w), xmax = max(0, max
 * w), s = fp16(fp32((xmax - xmin) / maxq)) (0 -> 1, overflow -> 65504),
 * z = clamp(rne(-xmin / s), 0, maxq) (with p->sym: s = fp16(fp32(max(-xmin,
 * xmax) / (2^(bits-1) - 1))), same 0 and overflow rules, z = 2^(bits-1));
 * then q = clamp(rne(w / s) + z, 0, maxq),
 * dq = s (q - z), e = (w - dq) / U[k][k] and every later column j gets
 * w_j -= e U[k][j].  Decisions are taken in fp32; the working copy is fp32.
 *
 *   W         device, d_out x d_in of w_dtype, row stride ld_w (elements).
 *   U, perm   from gptq_prepare_hinv.  perm is required when p->act_order is
 *             set (GPTQ_EINVAL otherwise: U is then in permuted order); NULL
 *             with act_order == 0 means the natural order.
 *   codes     device uint8 [batch][d_out][d_in], ORIGINAL column order.
 *   scales    device uint16 [batch][d_out][d_in / g]: fp16 bit patterns,
 *             groups in quantization order (static_groups: original order).
 *   zeros     device uint8 [batch][d_out][d_in / g].
 *   g_idx     device int32 [batch][d_in]: group of each original column
 *             (static_groups: c / g).
 *   Q_opt     optional device fp32 [batch][d_out][d_in]: dequantized weights in
 *             the original column order (the listing's return value), or NULL.
 * Batch entries are independent layers with the same shape (e.g. experts). */
gptq_status gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t d_out, int64_t d_in,
                                int64_t ld_w, int64_t batch, const float* U, const int32_t* perm,
                                const gptq_params* p, uint8_t* codes, uint16_t* scales,
                                uint8_t* zeros, int32_t* g_idx, float* Q_opt, void* workspace,
                                size_t ws_bytes, void* stream);

/* 4-bit packing ("INT4/INT8 量化推理", section 一: 128 x 4 bit = 64 bytes):
 * packed[r][c/2] = codes[r][c] | codes[r][c+1] << 4 (low nibble = even column).
 * codes: device uint8 rows x cols (values 0..15, cols even); packed: device
 * uint8 rows x cols/2.  Also used for the zeros (rows x groups). */
gptq_status gptq_pack_int4(const uint8_t* codes, int64_t rows, int64_t cols, uint8_t* packed,
                           void* stream);

/* Dense little-endian bit stream per row for `bits` in 2..8: code c occupies
 * stream bits c*bits .. c*bits+bits-1, least significant first; stream bit i
 * is bit (i mod 8) of byte i/8.  (cols * bits) % 8 == 0; packed is
 * rows x cols*bits/8.
 * bits = 4 gives the same bytes as gptq_pack_int4; bits = 3 stores 128 codes
 * in 48 bytes. */
gptq_status gptq_pack_bits(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits,
                           uint8_t* packed, void* stream);

/* W4A16 consumer of the packed format ("INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍",
 * section 六: weights stay 4-bit, activations 16-bit; section 一: the stored
 * group):  Y[m][n] = sum_k X[m][col(k)] s[n][k/g] (q[n][k] - z[n][k/g]).
 *
 *   X        device, M x d_in activations of x_dtype (GPTQ_F16 or GPTQ_BF16),
 *            row stride ld_x (elements).  1 <= M <= 64 (larger M:
 *            GPTQ_EUNSUPPORTED).
 *   qweight  device uint8 [d_out][d_in / 2] as gptq_pack_int4 writes it (low
 *            nibble first), 16-byte aligned.  Packed column k is input channel
 *            col(k) = perm[k] when perm is given, else k.
 *   scales   device uint16 [d_out][d_in / g] fp16 bits; group of packed
 *            column k is k / g.
 *   zeros    device uint8 [d_out][d_in / g] (one byte per zero, 0..15).
 *   perm     device int32 [d_in] or NULL.  For a layer quantized in act-order
 *            with dynamic groups pass gptq_prepare_hinv's perm and pack the
 *            codes in that order (gptq_pack_int4_permuted); natural order and
 *            static groups need none (their groups are k / g already).
 *   group_size  g: a multiple of 128 dividing d_in (smaller: GPTQ_EUNSUPPORTED).
 *   Y        device fp32 M x d_out, row stride ld_y.
 *   workspace  device, at least gptq_workspace_size(GPTQ_OP_W4A16, NULL,
 *            d_out, d_in, M, 1) bytes; calls sharing one workspace must be
 *            stream-ordered.
 * Arithmetic: fp32 accumulation on MFMA; the codes enter exactly (as q - z in
 * fp16, or as 128 + q in bf16 with the 128 + z term taken off through the
 * chunk's activation sum), each 128-channel chunk's sum is scaled by its
 * group's fp16 scale.  Results are bitwise reproducible for a given shape. */
gptq_status gptq_w4a16_matmul(const void* X, int32_t x_dtype, int64_t M, int64_t d_in, int64_t ld_x,
                              const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                              const int32_t* perm, int64_t d_out, int32_t group_size, float* Y,
                              int64_t ld_y, void* workspace, size_t ws_bytes, void* stream);

/* gptq_w4a16_matmul without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * gptq_w4a16_matmul, bit for bit; the scratch the call needs lives in a
 * fixed device array inside the library (8519936 bytes per GPU, the largest
 * call: M = 64, d_in = 65536), held by each GPU the library runs on until the
 * process ends.  Allocates nothing and does not take part in
 * gptq_timing_enable's records.  Every call on a GPU uses that GPU's one
 * array, so calls that overlap in time on one GPU (distinct streams,
 * threads) race and give wrong results: order them on one stream. */
gptq_status gptq_w4a16_matmul_noalloc(const void* X, int32_t x_dtype, int64_t M, int64_t d_in, int64_t ld_x,
                                      const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                                      const int32_t* perm, int64_t d_out, int32_t group_size, float* Y,
                                      int64_t ld_y, void* stream);

/* gptq_pack_int4 of the codes' columns taken in the order perm (for the
 * W4A16 consumer of an act-order layer): packed[r][k/2] holds codes[r][perm[k]]
 * (low nibble = even k).  codes: device uint8 rows x cols; perm: device int32
 * [cols], a permutation of 0..cols-1; packed: device uint8 rows x cols/2. */
gptq_status gptq_pack_int4_permuted(const uint8_t* codes, int64_t rows, int64_t cols, const int32_t* perm,
                                    uint8_t* packed, void* stream);

/* Activation-aware per-channel scaling as a pre-pass to GPTQ (ipipp.com
 * page, section 二: each input channel's weights are multiplied by a scale
 * derived from the activations, chosen among candidates by the output error,
 * and divided back out in the previous layer; "INT4/INT8 量化推理：从 GPTQ 到
 * AWQ 的取舍", section 四: exact before rounding).  Three calls:
 *
 * gptq_abs_accumulate: A[b][c] += sum of |x| over the entry's rows of X, in
 *   fp64; arguments, gathering and workspace as gptq_hessian_accumulate
 *   (workspace from GPTQ_OP_ABS).  Zero A before the first call; a_c =
 *   A[c] / N with N the tokens seen.
 *
 * gptq_awq_search: for every candidate alpha (host array, 1..256 values in
 *   [0, 4]): s_c = fp32(max(A[c] / N, 1e-6)^alpha) (division and power in
 *   fp64; N read from the device count n_tokens, which must be > 0);
 *   the residual W - RTN(W diag(s)) diag(s)^-1 with the path's group
 *   quantizer (p->bits, p->group_size, p->sym; w s rounded to fp32, the
 *   dequantized value divided back by s in fp32); its output error
 *   err[j] = ||residual Xs^T||_F^2 on the sample Xs (n_s x d_in rows of
 *   xs_dtype, row stride ld_xs), accumulated in fp64 from fp32 MFMA tiles of
 *   split-bf16 operands.  Then best = the first index of the smallest error
 *   and s_out = that candidate's scales.
 *     W        device, d_out x d_in of w_dtype, row stride ld_w.
 *     A        device fp64 [d_in] (gptq_abs_accumulate); n_tokens device
 *              int64 [1], the entry's Hessian count N.
 *     err_out  device fp64 [n_alpha]; s_out device fp32 [d_in];
 *     best_out device int32 [1].
 *     workspace  GPTQ_OP_AWQ_SEARCH bytes.
 *
 * gptq_awq_apply: the chosen scales applied in place to the Hessian state
 *   (S lower triangle incl. the diagonal: S_ij / (s_i s_j), computed in fp64
 *   and rounded to fp32; D_i / s_i^2) and W' = fp32(W s) written to W_out
 *   (device fp32 d_out x d_in, dense).  gptq_prepare_hinv and
 *   gptq_quantize_layer (with W_out, GPTQ_F32) then run unchanged; the codes
 *   describe W', and the layer's input must be divided by s (folded into the
 *   previous layer). */
gptq_status gptq_abs_accumulate(double* A, const void* X, int32_t x_dtype, int64_t n_rows, int64_t d_in,
                                int64_t ld_x, const int32_t* row_idx, const int64_t* row_ptr, int64_t batch,
                                void* workspace, size_t ws_bytes, void* stream);
gptq_status gptq_awq_search(const void* W, int32_t w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                            const double* A, const int64_t* n_tokens, const void* Xs, int32_t xs_dtype, int64_t n_s,
                            int64_t ld_xs, const gptq_params* p, const float* alphas, int32_t n_alpha,
                            double* err_out, float* s_out, int32_t* best_out, void* workspace, size_t ws_bytes,
                            void* stream);
gptq_status gptq_awq_apply(float* S, double* D, int64_t d_in, const float* s, const void* W, int32_t w_dtype,
                           int64_t d_out, int64_t ld_w, float* W_out, void* stream);

/* Forward of a quantized layer, for sequential calibration of a block
 * ("3. 模型量化技术(下)", section "GPTQ：基于二阶信息的后训练量化", pseudocode:
 * each layer is calibrated on its own inputs; here the next layer's inputs
 * are the already quantized layer's outputs):
 *   Y = round(act(X Q^T)), act 0 none, 1 ReLU, 2 SiLU (x / (1 + e^-x)),
 *   rounded to x_dtype (nearest even).
 *   X   device n_tok x d_in of x_dtype, row stride ld_x.
 *   Q   device fp32 d_out x d_in dequantized weights (gptq_quantize_layer's
 *       Q_opt), row stride ld_q.
 *   Y   device n_tok x d_out of x_dtype, row stride ld_y; must not overlap
 *       X, Q or the workspace.
 *   workspace  device, 256-byte aligned, at least gptq_workspace_size(
 *       GPTQ_OP_FORWARD, NULL, d_out, d_in, n_tok, 1) bytes (X and Q as
 *       16-bit terms); calls sharing one workspace must be stream-ordered.
 * fp32 accumulation on MFMA; d_in a multiple of 32.  fp16 X with 16-byte
 * aligned rows enters exactly, each row of Q as two fp16 terms of the row
 * scaled by a power of two (about 2^-22 relative); bf16 X with aligned rows
 * enters exactly, Q as two bf16 terms (about 2^-17); fp32 X or unaligned rows
 * are copied, X and Q each as two bf16 terms.  GPTQ_EINVAL on bad arguments
 * (checked before any GPU work), GPTQ_ENOMEM when the workspace is missing
 * or too small; n_tok = 0 does nothing. */
gptq_status gptq_layer_forward(const void* X, int32_t x_dtype, int64_t n_tok, int64_t d_in, int64_t ld_x,
                               const float* Q, int64_t d_out, int64_t ld_q, int32_t act, void* Y, int64_t ld_y,
                               void* workspace, size_t ws_bytes, void* stream);

/* Reference rates for measurement (not part of the quantization path): the
 * published peaks of a GPU are not what it sustains under a given load, so
 * the benchmark also measures two simple kernels on the same device.  Both
 * calls wait for their own launches (they synchronize the stream).
 *
 * gptq_probe_mfma: grids of 256 to 2048 workgroups of 4 waves (1 to 8 waves
 *   per SIMD), each wave issuing 4 * iters MFMAs with random operands on
 *   registers (kind 0: fp16 32x32x16, 1: bf16 32x32x16, 2: fp64 16x16x4,
 *   the same operands for every MFMA; kind 3: fp16, 4: bf16 32x32x16 with
 *   eight operand sets taken in turn, so every MFMA gets new input bits, and
 *   iters rounded up to even); writes the best rate over the grids (each the
 *   best of three timed launches) as TFLOP/s to *tflops_out (host).  sink:
 *   device scratch of gptq_probe_sink_bytes() bytes that receives each lane's
 *   sum.  EINVAL for any other kind.
 * gptq_probe_copy: dst = src for `bytes` (a multiple of 16; both 16-byte
 *   aligned device buffers, not overlapping) with a plain streaming kernel on
 *   grids of 1024 to 16384 workgroups; *gbs_out = read + write bytes per
 *   second / 1e9 of the fastest launch, *ms_out (optional) its duration. */
size_t gptq_probe_sink_bytes(void);
gptq_status gptq_probe_mfma(int32_t kind, int32_t iters, float* sink, double* tflops_out, void* stream);
gptq_status gptq_probe_copy(const void* src, void* dst, size_t bytes, double* gbs_out, double* ms_out,
                            void* stream);

/* Optional kernel timing for measurement.  When enabled, the library records
 * a pair of HIP events on the launch stream around every launch of the
 * kernels of `kind` (0 = Hessian MFMA product, 1 = fp64 diagonal, 2 = factor
 * kernels, 3 = block quantization, 4 = deferred update GEMM, 5 = packing,
 * 6 = working-copy preparation, 7 = reduction of split Hessian partials,
 * 8 / 9 = W4A16 staging / main kernel, 10 = |x| sums, 11 = scale search,
 * 12 = scale application, 13 = layer forward).  gptq_timing_read synchronizes those events
 * and reports the summed duration (ms) and launch count of `kind`; reset
 * drops all records.  Not thread safe; off by default. */
gptq_status gptq_timing_enable(int32_t on);
gptq_status gptq_timing_reset(void);
gptq_status gptq_timing_read(int32_t kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
