/*
 * qurl_w8a8.h -- C ABI of the MI355X (gfx950) W8A8 quantized linear used by a
 * quantized RL rollout actor ("QuRL: Efficient Reinforcement Learning with
 * Quantized Rollout").
 *
 * Sources, cited by page and section:
 *   [Notes/Framework]  paper-notes page, "Method > Overall framework": the old
 *                      actor theta_old is quantized to theta_hat_old for every
 *                      rollout.
 *   [Notes/UAQ]        same page, "Method > Key designs > UAQ": W X = (W/s)(sX),
 *                      s > 1 applied to W column-wise and to the activation
 *                      row-wise, mergeable into the preceding norm.
 *   [Notes/System]     same page, "Method > System integration": UAQ is a
 *                      one-time weight preprocessing; rollout runs on INT8/FP8
 *                      matrix-multiplication kernels.
 *   [Notes/Training]   same page, "Loss / training strategy": channel-wise
 *                      weight quantization, token-wise activation
 *                      quantization, INT8 or FP8, s = 1.5.
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout     Row-major. Weights W / codes Wq are [N, K] (torch.nn.Linear
 *            out x in, K contiguous); activations X / codes Xq are [M, K];
 *            outputs Y are [M, N]. Leading dimensions (ld*) count elements.
 * Pointers   All array pointers are DEVICE pointers (memory of the current
 *            HIP device). Matrices are 16-byte aligned, scale vectors 4-byte
 *            aligned. Codes Xq and Wq are dense (leading dimension K).
 * Dtypes     bf16 is passed as its 16-bit pattern (uint16); INT8 codes are
 *            int8; FP8 codes are OCP E4M3FN bytes (bias 7, max 448, no inf);
 *            scales and master weights are IEEE fp32.
 * Shapes     M, N >= 0 (0 makes the call a successful no-op); K >= 0 with
 *            K % 16 == 0; INT8 needs K <= 133144 so that K*127^2 < 2^31;
 *            the GEMM needs N*K and M*K below 2^31 - 2^16 (code matrices
 *            just under 2 GiB).
 *            ldx % 8 == 0, ldw % 4 == 0, any ldy >= N (ldy % 4 == 0 lets the
 *            epilogue store four outputs at a time).
 * Ownership  The caller allocates and owns every buffer, including the
 *            workspace. The library never allocates, frees or synchronizes.
 * Streams    `stream` is a hipStream_t passed as void* (NULL = the null
 *            stream). Every call only enqueues work on it and returns.
 * Errors     Arguments are validated on the host before anything is
 *            enqueued: a non-QR_OK status means nothing was launched.
 *            qr_last_error() returns a thread-local message for the last
 *            failure. Device faults surface at the caller's next
 *            synchronization, as for any asynchronous HIP work.
 * Finiteness Inputs must be finite; NaN/Inf inputs give unspecified codes.
 * Threads    Calls are reentrant; concurrent calls on different streams must
 *            not share a workspace.
 */
#ifndef QURL_W8A8_H
#define QURL_W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantized code type. */
enum { QR_INT8 = 0, QR_FP8_E4M3FN = 1 };

/* Output mode of qr_w8a8_gemm. */
enum {
  QR_OUT_BF16 = 0, /* dequantized bf16 Y */
  QR_OUT_RAW = 1   /* raw accumulators: int32 (INT8) or fp32 (FP8) */
};

/* Status codes. */
enum {
  QR_OK = 0,
  QR_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum, bad s */
  QR_ERR_UNSUPPORTED = -2, /* valid but not handled: K % 16, alignment, K too large */
  QR_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small */
  QR_ERR_HIP = -4,         /* a HIP call failed (message has the HIP error) */
  QR_ERR_NO_DEVICE = -5    /* no HIP device is visible */
};

/*
 * qr_quantize_weights_uaq -- theta_old -> theta_hat_old with UAQ
 *   [Notes/UAQ], [Notes/Framework], [Notes/Training], [Notes/System].
 *
 * For every output channel n (row of W):
 *   W'[n,k]    = fl32(W[n,k] / s)                 (UAQ: the stored weight is W/s)
 *   a_n        = max_k |W'[n,k]|
 *   scale_w[n] = fl32(a_n / Q)                    Q = 127 (INT8) or 448 (FP8)
 *   INT8: Wq   = clamp(round_half_even(fl32(W' / scale_w[n])), -127, 127)
 *   FP8:  Wq   = E4M3FN_round_half_even(clamp(fl32(W' / scale_w[n]), -448, 448))
 *   a_n == 0 gives scale_w[n] = 0 and all-zero codes.
 * s = 1.5 is the pages' value; pass s = 1 to re-quantize weights that were
 * already divided by s (the per-RL-step refresh).
 *
 *   W        [N, ldw] fp32 master weights (read).
 *   s        UAQ factor, finite and > 0.
 *   qt       QR_INT8 or QR_FP8_E4M3FN.
 *   Wq       [N, K] codes (written).
 *   scale_w  [N] fp32 per-channel scales (written).
 *   W_scaled optional [N, ldw] fp32 output of W' (NULL to skip). It may equal
 *            W to reparameterize in place (the one-time preprocessing).
 *   gamma    optional [K] fp32 gain of the norm that feeds this linear; if
 *            non-NULL it is multiplied by s in place (gamma' = fl32(gamma*s)),
 *            which folds the activation-side s into the norm. Do this once,
 *            at the one-time reparameterization, and only for one of the
 *            linears that share the norm.
 *   beta     optional [K] fp32 LayerNorm bias, multiplied by s like gamma.
 */
int qr_quantize_weights_uaq(const float* W, int64_t N, int64_t K, int64_t ldw, float s, int qt,
                            void* Wq, float* scale_w, float* W_scaled, float* gamma, float* beta,
                            void* stream);

/*
 * qr_requantize_weights -- the per-RL-step refresh theta_old -> theta_hat_old
 * [Notes/Framework] of a stored parameter that is already W' = W / s, with,
 * per output channel, the number of codes the update changed [Notes/UAQ:
 * updates far below one step leave almost every code unchanged].
 *
 * Per output channel n of Wp (s = 1, so W' itself is quantized):
 *   scale_w[n] = fl32(max_k |Wp[n,k]| / Q), codes from fl32(Wp[n,k] / scale_w[n])
 * exactly as qr_quantize_weights_uaq with s = 1. If row_flips is non-NULL,
 * Wq must hold the previous codes on entry: every code is compared with the
 * one it overwrites and row_flips[n] receives the number of positions of
 * row n whose value changed (INT8: any byte change; E4M3FN: any byte change
 * except +0 <-> -0). Counts are written, not accumulated, with plain stores
 * (no atomics: many waves adding to one device counter serialize).
 *
 *   Wp        [N, ldw] fp32 stored parameters (read).
 *   qt        QR_INT8 or QR_FP8_E4M3FN.
 *   Wq        [N, K] codes (previous codes read when counting, new codes written).
 *   scale_w   [N] fp32 per-channel scales (written).
 *   row_flips NULL, or [N] uint32 per-channel change counts (written).
 * Errors as for qr_quantize_weights_uaq; nothing is launched on an error.
 */
int qr_requantize_weights(const float* Wp, int64_t N, int64_t K, int64_t ldw, int qt, void* Wq,
                          float* scale_w, uint32_t* row_flips, void* stream);

/*
 * qr_quantize_act_per_token -- token-wise absmax quantization [Notes/Training].
 *
 * For every token m (row of X), with x = X[m,:] widened exactly to fp32:
 *   a_m        = max_k |x_k|,  t_m = fl32(a_m / Q)
 *   codes      as for the weights, from fl32(x_k / t_m)
 *   scale_x[m] = fl32(t_m * act_mult)
 * act_mult carries the UAQ factor onto the activation side of a linear whose
 * input does not come from a norm that absorbed s ([Notes/UAQ]): pass s there
 * and 1 for norm-fed linears. (With absmax quantization the codes of s*x equal
 * those of x, so s only multiplies the scale.)
 *
 *   X        [M, ldx] bf16 bit patterns (read).
 *   act_mult finite, > 0.
 *   Xq       [M, K] codes (written); scale_x [M] fp32 (written).
 */
int qr_quantize_act_per_token(const void* X, int64_t M, int64_t K, int64_t ldx, float act_mult,
                              int qt, void* Xq, float* scale_x, void* stream);

/* Norm kinds of qr_norm_quant. */
enum { QR_NORM_RMS = 0, QR_NORM_LAYER = 1 };

/*
 * qr_norm_quant -- the norm that produces a linear's input, with the UAQ
 * factor s merged into its gain and bias [Notes/UAQ], fused with the
 * token-wise quantization [Notes/Training] of its output: one pass over H,
 * the normalized values never reach memory.
 *
 * For every token m, with h = H[m,:] widened exactly to fp32 and K = row length:
 *   QR_NORM_RMS:   ms = sum_k h_k^2 / K                       (float64)
 *                  r  = fl32(1 / sqrt(ms + eps))              (float64, rounded once)
 *                  y_k = fl32(fl32(h_k * r) * gamma[k])
 *   QR_NORM_LAYER: mu = fl32(sum_k h_k / K)                   (float64, rounded once)
 *                  ms = sum_k (h_k - mu)^2 / K                (float64)
 *                  r  = fl32(1 / sqrt(ms + eps))
 *                  y_k = fl32(fl32(fl32(h_k - mu) * r) * gamma[k])
 *   with beta: y_k = fl32(y_k + beta[k]).
 *   Codes and scale_x[m] = fl32(max_k |y_k| / Q) as qr_quantize_act_per_token
 *   with act_mult = 1 (s is already in gamma and beta).
 * The float64 sums may be taken in any order: r is the same fp32 value unless
 * the exact value lies within about 2^-45 (relative) of an fp32 rounding
 * boundary.
 *
 *   H        [M, ldh] bf16 bit patterns (read).
 *   norm     QR_NORM_RMS or QR_NORM_LAYER.
 *   gamma    [K] fp32 folded gain gamma*s (e.g. from qr_quantize_weights_uaq's
 *            fold); 16-byte aligned. beta: NULL or [K] fp32 folded bias beta*s.
 *   eps      finite, >= 0.
 *   Xq       [M, K] codes (written); scale_x [M] fp32 (written).
 * K <= 32768 (rows are held in registers). Errors as qr_quantize_act_per_token.
 */
int qr_norm_quant(const void* H, int64_t M, int64_t K, int64_t ldh, int norm, const float* gamma,
                  const float* beta, float eps, int qt, void* Xq, float* scale_x, void* stream);

/*
 * qr_silu_mul_quant -- the input of the down projection, SiLU(gate) * up,
 * fused with its token-wise quantization [Notes/Training]; its scale carries
 * the UAQ factor through act_mult = s ([Notes/UAQ]: no norm produces it).
 *
 *   a[m,n] = fl32(g * u / (1 + exp(-g))) evaluated in float64,
 *            g = G[m,n], u = U[m,n] (bf16, exact in float64)
 *   codes and scale_x[m] = fl32(fl32(max_n |a[m,n]| / Q) * act_mult) as
 *   qr_quantize_act_per_token.
 * The device exp and the host's may differ in the last float64 bit, which
 * changes a only where the exact value lies within about 2^-50 (relative) of
 * an fp32 rounding boundary.
 *
 *   G, U     [M, ldg] / [M, ldu] bf16 (read): e.g. the two halves of one
 *            stacked gate+up GEMM output, G = Y, U = Y + N, ldg = ldu = 2N.
 *   act_mult finite, > 0.
 *   Xq       [M, N] codes (written); scale_x [M] fp32 (written).
 * N <= 32768. Errors as qr_quantize_act_per_token.
 */
int qr_silu_mul_quant(const void* G, const void* U, int64_t M, int64_t N, int64_t ldg, int64_t ldu,
                      float act_mult, int qt, void* Xq, float* scale_x, void* stream);

/*
 * qr_acr_tis_loss -- the trainer-side objective that goes with the quantized
 * rollout: ACR's adaptive clipping range with truncated importance sampling
 * [Notes/ACR], per token, as a loss, with its gradient and deterministic sums.
 *
 * For every token t (fp32 arithmetic):
 *   R = exp(logp - logp_prox)         ratio to the full-precision old actor
 *   r = exp(logp_prox - logp_behav)   full-precision over the quantized actor
 *                                     that sampled the token
 *   w = min(r, C);  lo = 1 - eps;  hi = (1 + eps) / r
 *   term = min(R A, min(max(R, lo), hi) A)
 *   loss[t] = -w term;  grad[t] = d loss[t] / d logp[t] = -w R A where the
 *   unclipped branch is the minimum, else 0. Masked tokens: 0, not counted.
 *   sums = {sum of loss over valid tokens, valid tokens, clipped valid tokens}
 *   (float64, from per-block partials added in a fixed order, strided runs
 *   then a pairwise tree: the same bits on every run). The mean loss is
 *   sums[0] / sums[1].
 *
 *   logp, logp_prox, logp_behav, adv  [n] fp32, 16-byte aligned (read).
 *   mask     [n] uint8, nonzero = response token; 4-byte aligned (read).
 *   eps      in [0, 1);  C  > 0 (may be +inf: no truncation).
 *   loss     [n] fp32 (written);  grad  NULL or [n] fp32 (written).
 *   sums     [3] float64 (written).
 *   workspace  at least qr_workspace_size("qr_acr_tis_loss", n, 0, 0, 0)
 *            bytes, 8-byte aligned; contents on entry irrelevant.
 * n < 2^31. Errors as for the other entry points.
 */
int qr_acr_tis_loss(const float* logp, const float* logp_prox, const float* logp_behav,
                    const float* adv, const uint8_t* mask, int64_t n, float eps, float C,
                    float* loss, float* grad, double* sums, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * qr_mx_quantize -- block-wise FP8: every 32 consecutive elements of a row
 * share one power-of-two scale (the block-wise FP8 variant the pages cite,
 * [fugumt] "Related papers"; block of 32 with E8M0 scales as the gfx950
 * scaled MFMA applies them).
 *
 * For every row r and block b of A (values v widened exactly to fp32):
 *   X = the smallest integer with max |v| <= 448 * 2^X (clamped to
 *       [-127, 127]; an all-zero block gives -127); the scale byte of block b
 *       of row r is X + 127 (stored as below);
 *   codes[r, 32 b + i] = E4M3FN(min(max(fl32(v_i * 2^-X), -448), 448)),
 *       nearest, ties to even, sign kept on zero.
 *
 *   A        [R, lda] fp32 (src_bf16 = 0) or bf16 bit patterns (src_bf16 = 1).
 *   K        multiple of 32.
 *   codes    [R, K] E4M3FN bytes (written).
 *   scales   E8M0 bytes in panels of 128 elements of K, [ceil(K/128)][R][4]:
 *            the byte of block b of row r is at ((b / 4) R + r) 4 + b % 4
 *            (written; the unused bytes of a partial last panel are left as
 *            they are). A row's four bytes for one 128-element K step are
 *            adjacent and a run of rows' bytes for that step is contiguous,
 *            which is what the GEMM copies per step.
 * Errors as for qr_quantize_act_per_token.
 */
int qr_mx_quantize(const void* A, int64_t R, int64_t K, int64_t lda, int src_bf16, void* codes,
                   uint8_t* scales, void* stream);

/*
 * qr_mx_gemm -- product of block-wise FP8 operands:
 *   acc[m,n] = sum_b 2^(Xx[m,b] + Xw[n,b]) sum_{k in block b} x[m,k] w[n,k]
 *   (the gfx950 scaled MFMA applies the block scales; products within a
 *   group of k are added at the FP8 MFMA's reduced precision, groups in
 *   fp32, as for qr_w8a8_gemm's FP8 path).
 *   out = QR_OUT_BF16: Y[m,n] = bf16_rne(acc);  QR_OUT_RAW: Y = acc (fp32).
 *
 *   Xq, sx   [M, K] codes and the tokens' E8M0 scales ([K/128][M][4] panels,
 *            as qr_mx_quantize writes them).
 *   Wq, sw   [N, K] codes and the weights' E8M0 scales ([K/128][N][4]).
 *            Xq, Wq, sx, sw and Y start on 16-byte boundaries (else
 *            QR_ERR_UNSUPPORTED).
 *   K        multiple of 128; code matrices below 2^31 - 2^16 bytes.
 *   Y        [M, ldy] bf16 or fp32 (written).
 */
int qr_mx_gemm(const void* Xq, const uint8_t* sx, const void* Wq, const uint8_t* sw, int64_t M,
               int64_t N, int64_t K, int out, void* Y, int64_t ldy, void* stream);

/*
 * qr_w8a8_gemm -- quantized product and dequantization epilogue
 *   [Notes/System] (INT8/FP8 matmul), [Notes/Training].
 *
 *   acc[m,n] = sum_k Xq[m,k] * Wq[n,k]
 *              INT8: exact int32.  FP8: sums of E4M3FN products formed by
 *              the gfx950 MFMA unit, which adds the products of a group of
 *              k at reduced precision (bits far below the group's largest
 *              product are dropped) and accumulates groups in fp32; the
 *              result is deterministic for a given shape and plan.
 *   out = QR_OUT_BF16: Y[m,n] = bf16_rne(fl32(fl32(fl32(acc) * scale_x[m]) * scale_w[n]))
 *   out = QR_OUT_RAW : Y[m,n] = acc (int32 or fp32), for parity checks.
 *
 *   Y        [M, ldy] bf16, int32 or fp32 (written).
 *   workspace    device scratch of at least qr_workspace_size("qr_w8a8_gemm",
 *                M, N, K, qt) bytes, 256-byte aligned; may be NULL when that
 *                size is 0 (no K split for this shape). It holds the split-K
 *                partial sums; its contents on entry do not matter and are
 *                undefined on return. Calls that may run at the same time
 *                (different streams) must not share it.
 */
int qr_w8a8_gemm(const void* Xq, const float* scale_x, const void* Wq, const float* scale_w,
                 int64_t M, int64_t N, int64_t K, int qt, int out, void* Y, int64_t ldy,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * qr_w8a8_gemm_quant -- one linear of a decode chain in one launch: the
 * quantized product and its dequantization epilogue [Notes/System],
 * [Notes/Training], and the token-wise quantization [Notes/Training] of a
 * column range of its bf16 output, the next linear's input (the activation
 * side of UAQ [Notes/UAQ] rides on q_act_mult as for
 * qr_quantize_act_per_token).
 *
 *   Y         = qr_w8a8_gemm(..., QR_OUT_BF16)                  [M, ldy] bf16
 *   Xq_next, scale_x_next
 *             = qr_quantize_act_per_token(Y[:, q_col0 : q_col0 + q_cols],
 *                                         q_act_mult)           [M, q_cols], [M]
 *   bit for bit the results of those two calls. q_cols = 0 quantizes
 *   nothing (Xq_next and scale_x_next are not used).
 * By default the call launches the GEMM and then, for a plan that splits K
 * (qr_gemm_plan) with q_cols > 0 and N a multiple of 8 up to 16384, one
 * kernel that adds the partial sums, applies the epilogue and quantizes the
 * column range; otherwise the GEMM (and its split-K kernel) and the
 * quantizer. With qr_set_fuse_override(1), where the plan allows (all
 * blocks of the grid resident on the GPU at once, M <= 4096, N, ldy
 * multiples of 4, Y 16-byte aligned) the split-K sum and the quantization
 * run inside the GEMM launch behind grid-wide barriers instead (one launch;
 * measured slower than the separate launches on the 7B- and 32B-shaped
 * linears, so it is not the default).
 *
 *   Xq, scale_x, Wq, scale_w, M, N, K, qt, Y, ldy   as qr_w8a8_gemm.
 *   q_col0, q_cols  column range of Y to quantize: multiples of 16 (the
 *             next linear's K), q_col0 + q_cols <= N; ldy % 8 == 0 when
 *             q_cols > 0.
 *   q_act_mult      finite, > 0 (the next linear's act_mult).
 *   Xq_next   [M, q_cols] codes (written), 16-byte aligned.
 *   scale_x_next    [M] fp32 (written).
 *   workspace at least qr_workspace_size("qr_w8a8_gemm_quant", M, N, K, qt)
 *             bytes, 256-byte aligned. Its first 64 KiB are barrier and
 *             per-token maximum words: they must be zero before the first
 *             call that uses this workspace, and every call leaves them
 *             ready for the next one (zero the buffer once when it is
 *             allocated; do not share it with calls of other entry points,
 *             which use a workspace from its start). The rest holds split-K
 *             partial sums. Calls that may run at the same time (different
 *             streams) must not share it.
 */
int qr_w8a8_gemm_quant(const void* Xq, const float* scale_x, const void* Wq, const float* scale_w,
                       int64_t M, int64_t N, int64_t K, int qt, void* Y, int64_t ldy, int64_t q_col0,
                       int64_t q_cols, float q_act_mult, void* Xq_next, float* scale_x_next,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * qr_linear_fused -- the per-linear call of a rollout engine:
 *   qr_quantize_act_per_token followed by qr_w8a8_gemm(out = QR_OUT_BF16),
 *   with the activation codes and scales kept in the workspace.
 *
 *   X        [M, ldx] bf16 (read); Y [M, ldy] bf16 (written).
 *   workspace    at least qr_workspace_size("qr_linear_fused", M, N, K, qt)
 *                bytes (never 0 when M, N > 0), 256-byte aligned scratch:
 *                split-K partial sums, then the activation codes and scales.
 *
 *   Decode steps of a few tokens (M x K <= 8192, e.g. 1 or 2 tokens of a
 *   3584-wide input; with qr_set_small_m_override up to M <= 4 and
 *   M x K <= 20480) run as one launch whose blocks quantize X themselves
 *   into on-chip memory and split K among their waves: the workspace is
 *   then not touched (it is still required), no codes are written to
 *   memory, and the result is the same (INT8: the same bits; FP8: the fp32
 *   sums of the waves' partial accumulators are added in a fixed order, so
 *   the bf16 output may differ from the two-call path within the FP8
 *   accumulation bound). qr_set_small_m_override selects or disables it.
 */
int qr_linear_fused(const void* X, int64_t ldx, float act_mult, const void* Wq, const float* scale_w,
                    int64_t M, int64_t N, int64_t K, int qt, void* Y, int64_t ldy,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qr_linear_fused_noalloc -- qr_linear_fused for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, with the
 * workspace (split-K partial sums, activation codes and scales) in a fixed
 * 48 MiB device array owned by the library, one per GPU, held until the
 * process ends. No call allocates or frees memory; the first call on a
 * device looks up that device's array (hipGetSymbolAddress).
 *   Arguments as qr_linear_fused, without the workspace.
 *   Shapes whose qr_workspace_size("qr_linear_fused", ...) exceeds 48 MiB
 *   return QR_ERR_WORKSPACE with nothing launched (e.g. up to 512 tokens for
 *   the 7B- and 32B-shaped linears fit).
 *   Every call on one GPU uses that GPU's one array, so calls that may run at
 *   the same time on one GPU (different streams) race and must not be made;
 *   calls ordered on one stream are safe. Nothing in the array needs to be
 *   zero: each call writes what it later reads.
 */
int qr_linear_fused_noalloc(const void* X, int64_t ldx, float act_mult, const void* Wq,
                            const float* scale_w, int64_t M, int64_t N, int64_t K, int qt,
                            void* Y, int64_t ldy, void* stream);

/*
 * qr_workspace_size -- bytes of workspace needed by `fn` ("qr_w8a8_gemm",
 * "qr_w8a8_gemm_quant" or "qr_linear_fused") for this shape; 0 if none. For "qr_acr_tis_loss" M is
 * the token count n (N, K and qt are ignored). Pure host function: it
 * depends only on its arguments (and on qr_set_plan_override). Returns
 * (size_t)-1 for an unknown fn or invalid sizes.
 */
size_t qr_workspace_size(const char* fn, int64_t M, int64_t N, int64_t K, int qt);

/*
 * qr_gemm_plan -- report the kernel plan qr_w8a8_gemm uses for a shape:
 *   *tile    index of the tile configuration (see qr_tile_name),
 *   *splitk  number of K splits (1 = none),
 *   *rows    output channels (weight rows) per tile, a multiple of 8 no
 *            larger than the configuration's tile height.
 * Pure host function; returns QR_OK or QR_ERR_INVALID_ARG.
 */
int qr_gemm_plan(int64_t M, int64_t N, int64_t K, int qt, int* tile, int* splitk, int* rows);

/* Name of tile configuration `tile` (static string) or NULL if out of range. */
const char* qr_tile_name(int tile);

/* Number of tile configurations. */
int qr_num_tiles(void);

/*
 * qr_set_plan_override -- tuning and test hook: force tile configuration
 * `tile`, `splitk` splits (0 = automatic) and `rows` weight rows per tile
 * (0 = the tile height; else a multiple of 8 no larger than it) for every
 * later qr_w8a8_gemm / qr_linear_fused / qr_workspace_size / qr_gemm_plan
 * call made by the calling thread (tile < 0 restores automatic planning).
 * The override is thread-local: other threads keep their own plans. Set it
 * before querying qr_workspace_size, and keep it until the GEMM call, since
 * the workspace a plan needs depends on it. Meant for benchmarks and tests.
 * Returns QR_OK or QR_ERR_INVALID_ARG.
 */
int qr_set_plan_override(int tile, int splitk, int rows);

/*
 * qr_set_small_m_override -- tuning and test hook for the one-launch
 * decode path of qr_linear_fused (and qr_linear_fused_noalloc): rf = 0
 * takes it where it is the faster path (M x K <= 8192), rf = -1 never,
 * rf = 1..5 wherever it can run (M <= 4, M x K <= 20480) with blocks of
 * 16 * rf output channels. A qr_set_plan_override tile also disables the
 * path. Thread-local like qr_set_plan_override; meant for benchmarks and
 * tests. Returns QR_OK or QR_ERR_INVALID_ARG.
 */
int qr_set_small_m_override(int rf);

/*
 * qr_set_fuse_override -- tuning and test hook for qr_w8a8_gemm_quant:
 * mode 0 (the default) runs its separate launches, mode 1 its one-launch
 * grid-barrier path wherever the plan allows. The results are the same.
 * Thread-local like qr_set_plan_override; meant for benchmarks and tests.
 * Returns QR_OK or QR_ERR_INVALID_ARG for another mode.
 */
int qr_set_fuse_override(int mode);

/*
 * Measurement helpers (not part of the linear): the peaks the chip reaches,
 * against which the GEMMs' roofline fractions are also reported.
 *
 * qr_probe_read -- read `bytes` (a multiple of 16) of device memory at `buf`
 *   (16-byte aligned) once with 16-byte non-temporal loads; block b writes
 *   one XOR word to sink[b]. sink holds at least sink_words >= 1024 uint32
 *   (device memory).
 *   bytes / kernel time is the memory read rate; use a buffer well past the
 *   256 MB Infinity Cache to measure HBM.
 * qr_probe_mfma -- `blocks` blocks of 8 waves; every wave runs `iters`
 *   rounds of 8 independent dense MFMAs on register operands (qt = QR_INT8:
 *   v_mfma_i32_32x32x32_i8, 65536 ops each; QR_FP8_E4M3FN:
 *   v_mfma_scale_f32_32x32x64_f8f6f4, 131072 ops each) and writes one word
 *   per wave to sink[8 b + w] (device, >= 8 * blocks uint32). Wave 0 of block
 *   b writes its shader-clock counter and the constant-rate wall clock at
 *   start and end to ticks[4 b + 0..3] (device, >= 4 * blocks uint64), and
 *   *wall_khz (host) receives the wall clock's rate, so that
 *   (t1 - t0) / (w1 - w0) * wall_khz is the shader clock in kHz.
 *   blocks in [1, 65536], iters in [1, 2^24].
 * qr_probe_copy_stream -- the operand copies of one LDS-DMA GEMM tiling with
 *   no matrix work: the blocks, copies, LDS ring, waits and per-step
 *   barriers that qr_w8a8_gemm runs for tile `tile` (4: 256x256 tiles,
 *   2-slot ring, non-temporal weight copies; 8: 192x128 tiles, 4-slot ring;
 *   10: 192x256 tiles, 2-slot ring, non-temporal weight copies) with `rows` weight rows per tile (a multiple of 8 up to the tile height,
 *   as qr_gemm_plan reports it), without split K, over the codes Wq (N rows)
 *   and Xq (M rows) of K bytes each (device, K a multiple of 128). Its time
 *   is what that tiling's copy pipeline alone takes. Row r of Xq starts at
 *   byte r * ldx, row r of Wq at r * ldw (ldw, ldx >= K, multiples of 16; the
 *   GEMM's layout is ldw = ldx = K). Variants, by `flags`:
 *   QR_PROBE_PANEL reads Wq as K panels, the 128 bytes of K step k of row r
 *   at byte (k * N + r) * 128 (ldw ignored), so that each step of a tile is
 *   one contiguous block; QR_PROBE_NO_BARRIER drops the barrier per K step
 *   (each wave waits only for its own copies); QR_PROBE_RESIDENT copies the
 *   bytes of K step 0 at every step (the same copies, waits and barriers,
 *   the operands resident in L2 after the first step), the copy pipeline's
 *   rate when no miss reaches HBM. Flags combine. Block b (tile
 *   n = b / tiles_m, token tile m = b % tiles_m, tiles_m = ceil(M / tile
 *   width)) writes to sink[b] the XOR of the four 32-bit words of the first
 *   16 bytes of the last K step copied (K / 128 - 1; 0 with
 *   QR_PROBE_RESIDENT) of weight row n * rows and of token row m * width, as
 *   they arrived in LDS, so the copies can be checked. sink: device,
 *   >= ceil(N / rows) * tiles_m words. QR_ERR_INVALID_ARG for another tile,
 *   unknown flags, bad sizes or strides or a short sink;
 *   QR_ERR_UNSUPPORTED for a code buffer of 2^31 - 2^16 bytes or more.
 */
int qr_probe_read(const void* buf, size_t bytes, uint32_t* sink, int64_t sink_words, void* stream);
enum { QR_PROBE_PANEL = 1, QR_PROBE_NO_BARRIER = 2, QR_PROBE_RESIDENT = 4 };
int qr_probe_copy_stream(int tile, const void* Wq, int64_t N, int64_t ldw, const void* Xq, int64_t M,
                         int64_t ldx, int64_t K, int rows, int flags, uint32_t* sink, int64_t sink_words,
                         void* stream);
int qr_probe_mfma(int qt, int blocks, int iters, uint32_t* sink, uint64_t* ticks, int* wall_khz,
                  void* stream);

/* Thread-local message describing the last non-QR_OK status ("" if none). */
const char* qr_last_error(void);

/* Library version string. */
const char* qr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QURL_W8A8_H */
