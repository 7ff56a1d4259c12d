// C ABI of the W8A8 linear (declared and documented in include/qurl_w8a8.h).
//
// Every entry point validates its arguments on the host first and returns an
// error before anything is enqueued; then it enqueues its kernels on the
// caller's stream and returns without synchronizing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "qr_internal.h"
#include "qurl_w8a8.h"

namespace {

thread_local std::string g_err;
// Plan override of qr_set_plan_override (a tuning and test hook): per thread,
// so a sweep on one thread never changes the plans, or the workspace sizes,
// that calls on other threads see.
thread_local int g_force_tile = -1;
thread_local int g_force_splitk = 0;
thread_local int g_force_rows = 0;
thread_local int g_small_m = 0;  // small-token path: 0 automatic, -1 off, 1..5 rows / 16
thread_local int g_fuse = 0;     // qr_w8a8_gemm_quant: 0 separate launches, 1 one launch

constexpr int64_t kMaxKInt8 = 133144;  // K * 127^2 < 2^31
constexpr int64_t kMaxDim = (int64_t)1 << 31;
// GEMM: 32-bit buffer offsets; 2^31 (minus at most 3 KB of copy bias) marks
// out-of-range rows, so code matrices stay below 2^31 - 2^16 bytes.
constexpr int64_t kMaxCodeBytes = ((int64_t)1 << 31) - ((int64_t)1 << 16);

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return QR_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  const int code =
      (e == hipErrorNoDevice || e == hipErrorInvalidDevice) ? QR_ERR_NO_DEVICE : QR_ERR_HIP;
  return fail(code, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool valid_qt(int qt) { return qt == QR_INT8 || qt == QR_FP8_E4M3FN; }

// Shape checks common to every call. Returns QR_OK or an error (g_err set).
int check_shape(const char* fn, int64_t M, int64_t N, int64_t K, int qt) {
  if (!valid_qt(qt)) return fail(QR_ERR_INVALID_ARG, "%s: unknown qtype %d", fn, qt);
  if (M < 0 || N < 0 || K < 0)
    return fail(QR_ERR_INVALID_ARG, "%s: negative size (M=%lld N=%lld K=%lld)", fn, (long long)M,
                (long long)N, (long long)K);
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(QR_ERR_UNSUPPORTED, "%s: size >= 2^31", fn);
  if (K % 16 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (qt == QR_INT8 && K > kMaxKInt8)
    return fail(QR_ERR_UNSUPPORTED, "%s: K=%lld > %lld would overflow the int32 accumulator", fn,
                (long long)K, (long long)kMaxKInt8);
  return QR_OK;
}

}  // namespace

namespace qr {

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_error(hipError_t e, const char* what) { return hip_status(e, what); }

}  // namespace qr


extern "C" {

const char* qr_last_error(void) { return g_err.c_str(); }

const char* qr_version(void) { return "qurl_w8a8 0.1.0 (gfx950)"; }

int qr_num_tiles(void) { return qr::num_tiles(); }

const char* qr_tile_name(int tile) {
  if (tile < 0 || tile >= qr::num_tiles()) return nullptr;
  return qr::tile_desc(tile).name;
}

int qr_set_plan_override(int tile, int splitk, int rows) {
  if (tile >= qr::num_tiles() || splitk < 0 || splitk > 1024)
    return fail(QR_ERR_INVALID_ARG, "qr_set_plan_override: tile %d / splitk %d out of range", tile,
                splitk);
  if (tile >= 0 && rows != 0 && (rows < 8 || rows % 8 != 0 || rows > qr::tile_desc(tile).BN))
    return fail(QR_ERR_INVALID_ARG,
                "qr_set_plan_override: rows %d must be 0 or a multiple of 8 in [8, %d]", rows,
                qr::tile_desc(tile).BN);
  g_force_tile = tile < 0 ? -1 : tile;
  g_force_splitk = tile < 0 ? 0 : splitk;
  g_force_rows = tile < 0 ? 0 : rows;
  return ok();
}

int qr_set_fuse_override(int mode) {
  if (mode != 0 && mode != 1)
    return fail(QR_ERR_INVALID_ARG, "qr_set_fuse_override: mode %d must be 0 or 1", mode);
  g_fuse = mode;
  return ok();
}

int qr_set_small_m_override(int rf) {
  if (rf < -1 || rf > qr::kSmallMaxRF)
    return fail(QR_ERR_INVALID_ARG, "qr_set_small_m_override: rf %d must be in [-1, %d]", rf,
                qr::kSmallMaxRF);
  g_small_m = rf;
  return ok();
}

int qr_gemm_plan(int64_t M, int64_t N, int64_t K, int qt, int* tile, int* splitk, int* rows) {
  int st = check_shape("qr_gemm_plan", M, N, K, qt);
  if (st != QR_OK) return st;
  if (!tile || !splitk || !rows)
    return fail(QR_ERR_INVALID_ARG, "qr_gemm_plan: null output pointer");
  const qr::GemmPlan p = qr::make_plan(M, N, K, qt, g_force_tile, g_force_splitk, g_force_rows);
  *tile = p.tile;
  *splitk = p.splitk;
  *rows = p.rows;
  return ok();
}

size_t qr_workspace_size(const char* fn, int64_t M, int64_t N, int64_t K, int qt) {
  if (!fn) return (size_t)-1;
  if (std::strcmp(fn, "qr_acr_tis_loss") == 0) {
    if (M < 0 || M >= kMaxDim) return (size_t)-1;
    return align256((size_t)qr::acr_blocks(M) * 3 * sizeof(double));
  }
  if (check_shape("qr_workspace_size", M, N, K, qt) != QR_OK) return (size_t)-1;
  const qr::GemmPlan p = qr::make_plan(M, N, K, qt, g_force_tile, g_force_splitk, g_force_rows);
  const size_t gemm = (M == 0 || N == 0) ? 0 : p.ws_bytes();
  if (std::strcmp(fn, "qr_w8a8_gemm") == 0) return gemm;
  if (std::strcmp(fn, "qr_w8a8_gemm_quant") == 0)
    return (M == 0 || N == 0) ? 0 : qr::kFuseHeaderBytes + p.part_bytes;
  if (std::strcmp(fn, "qr_linear_fused") == 0) {
    if (M == 0 || N == 0) return 0;
    return p.part_bytes + align256((size_t)M * (size_t)K) + align256((size_t)M * 4);
  }
  return (size_t)-1;
}

int qr_quantize_weights_uaq(const float* W, int64_t N, int64_t K, int64_t ldw, float s, int qt,
                            void* Wq, float* scale_w, float* W_scaled, float* gamma, float* beta,
                            void* stream) {
  const char* fn = "qr_quantize_weights_uaq";
  int st = check_shape(fn, 0, N, K, qt);
  if (st != QR_OK) return st;
  if (!std::isfinite(s) || !(s > 0.0f)) return fail(QR_ERR_INVALID_ARG, "%s: s must be finite and > 0", fn);
  if (ldw < K) return fail(QR_ERR_INVALID_ARG, "%s: ldw=%lld < K=%lld", fn, (long long)ldw, (long long)K);
  if (N > 0 && K > 0 && (!W || !Wq)) return fail(QR_ERR_INVALID_ARG, "%s: null W or Wq", fn);
  if (N > 0 && !scale_w) return fail(QR_ERR_INVALID_ARG, "%s: null scale_w", fn);
  if (ldw % 4 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: ldw must be a multiple of 4", fn);
  if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(W_scaled, 16) || !aligned(scale_w, 4) ||
      !aligned(gamma, 4) || !aligned(beta, 4))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for W, Wq, W_scaled)", fn);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (gamma || beta) {
    st = hip_status(qr::launch_fold_norm(gamma, beta, K, s, hs), fn);
    if (st != QR_OK) return st;
  }
  if (N == 0) return ok();
  return hip_status(qr::launch_weight_quant(W, N, K, ldw, s, qt, Wq, scale_w, W_scaled, hs), fn);
}

int qr_requantize_weights(const float* Wp, int64_t N, int64_t K, int64_t ldw, int qt, void* Wq,
                          float* scale_w, uint32_t* row_flips, void* stream) {
  const char* fn = "qr_requantize_weights";
  int st = check_shape(fn, 0, N, K, qt);
  if (st != QR_OK) return st;
  if (ldw < K) return fail(QR_ERR_INVALID_ARG, "%s: ldw=%lld < K=%lld", fn, (long long)ldw, (long long)K);
  if (N > 0 && K > 0 && (!Wp || !Wq)) return fail(QR_ERR_INVALID_ARG, "%s: null Wp or Wq", fn);
  if (N > 0 && !scale_w) return fail(QR_ERR_INVALID_ARG, "%s: null scale_w", fn);
  if (ldw % 4 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: ldw must be a multiple of 4", fn);
  if (!aligned(Wp, 16) || !aligned(Wq, 16) || !aligned(scale_w, 4) || !aligned(row_flips, 4))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for Wp, Wq; 4 for the rest)",
                fn);
  if (N == 0) return ok();
  (void)hipGetLastError();
  return hip_status(qr::launch_requant(Wp, N, K, ldw, qt, Wq, scale_w, row_flips,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_quantize_act_per_token(const void* X, int64_t M, int64_t K, int64_t ldx, float act_mult,
                              int qt, void* Xq, float* scale_x, void* stream) {
  const char* fn = "qr_quantize_act_per_token";
  int st = check_shape(fn, M, 0, K, qt);
  if (st != QR_OK) return st;
  if (!std::isfinite(act_mult) || !(act_mult > 0.0f))
    return fail(QR_ERR_INVALID_ARG, "%s: act_mult must be finite and > 0", fn);
  if (ldx < K) return fail(QR_ERR_INVALID_ARG, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
  if (M > 0 && K > 0 && (!X || !Xq)) return fail(QR_ERR_INVALID_ARG, "%s: null X or Xq", fn);
  if (M > 0 && !scale_x) return fail(QR_ERR_INVALID_ARG, "%s: null scale_x", fn);
  if (ldx % 8 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: ldx must be a multiple of 8", fn);
  if (!aligned(X, 16) || !aligned(Xq, 16) || !aligned(scale_x, 4))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for X, Xq)", fn);
  if (M == 0) return ok();
  (void)hipGetLastError();
  return hip_status(qr::launch_act_quant(X, M, K, ldx, act_mult, qt, Xq, scale_x,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_norm_quant(const void* H, int64_t M, int64_t K, int64_t ldh, int norm, const float* gamma,
                  const float* beta, float eps, int qt, void* Xq, float* scale_x, void* stream) {
  const char* fn = "qr_norm_quant";
  int st = check_shape(fn, M, 0, K, qt);
  if (st != QR_OK) return st;
  if (norm != QR_NORM_RMS && norm != QR_NORM_LAYER)
    return fail(QR_ERR_INVALID_ARG, "%s: unknown norm kind %d", fn, norm);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(QR_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if (ldh < K) return fail(QR_ERR_INVALID_ARG, "%s: ldh=%lld < K=%lld", fn, (long long)ldh, (long long)K);
  if (K > 32768) return fail(QR_ERR_UNSUPPORTED, "%s: K=%lld > 32768", fn, (long long)K);
  if (M > 0 && K > 0 && (!H || !Xq || !gamma))
    return fail(QR_ERR_INVALID_ARG, "%s: null H, Xq or gamma", fn);
  if (M > 0 && !scale_x) return fail(QR_ERR_INVALID_ARG, "%s: null scale_x", fn);
  if (K > 0 && ldh % 8 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: ldh must be a multiple of 8", fn);
  if (!aligned(H, 16) || !aligned(Xq, 16) || !aligned(gamma, 16) || !aligned(beta, 16) ||
      !aligned(scale_x, 4))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for H, Xq, gamma, beta)", fn);
  if (M == 0) return ok();
  (void)hipGetLastError();
  return hip_status(qr::launch_norm_quant(H, M, K, ldh, norm, gamma, beta, eps, qt, Xq, scale_x,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_silu_mul_quant(const void* G, const void* U, int64_t M, int64_t N, int64_t ldg, int64_t ldu,
                      float act_mult, int qt, void* Xq, float* scale_x, void* stream) {
  const char* fn = "qr_silu_mul_quant";
  int st = check_shape(fn, M, 0, N, qt);
  if (st != QR_OK) return st;
  if (!std::isfinite(act_mult) || !(act_mult > 0.0f))
    return fail(QR_ERR_INVALID_ARG, "%s: act_mult must be finite and > 0", fn);
  if (ldg < N || ldu < N)
    return fail(QR_ERR_INVALID_ARG, "%s: ldg=%lld / ldu=%lld < N=%lld", fn, (long long)ldg,
                (long long)ldu, (long long)N);
  if (N > 32768) return fail(QR_ERR_UNSUPPORTED, "%s: N=%lld > 32768", fn, (long long)N);
  if (M > 0 && N > 0 && (!G || !U || !Xq)) return fail(QR_ERR_INVALID_ARG, "%s: null G, U or Xq", fn);
  if (M > 0 && !scale_x) return fail(QR_ERR_INVALID_ARG, "%s: null scale_x", fn);
  if (N > 0 && (ldg % 8 != 0 || ldu % 8 != 0))
    return fail(QR_ERR_UNSUPPORTED, "%s: ldg and ldu must be multiples of 8", fn);
  if (!aligned(G, 16) || !aligned(U, 16) || !aligned(Xq, 16) || !aligned(scale_x, 4))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for G, U, Xq)", fn);
  if (M == 0) return ok();
  (void)hipGetLastError();
  return hip_status(qr::launch_silu_mul_quant(G, U, M, N, ldg, ldu, act_mult, qt, Xq, scale_x,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_acr_tis_loss(const float* logp, const float* logp_prox, const float* logp_behav,
                    const float* adv, const uint8_t* mask, int64_t n, float eps, float C,
                    float* loss, float* grad, double* sums, void* workspace, size_t ws_bytes,
                    void* stream) {
  const char* fn = "qr_acr_tis_loss";
  if (n < 0 || n >= kMaxDim) return fail(QR_ERR_INVALID_ARG, "%s: n=%lld out of range", fn, (long long)n);
  if (!std::isfinite(eps) || eps < 0.0f || eps >= 1.0f)
    return fail(QR_ERR_INVALID_ARG, "%s: eps must be in [0, 1)", fn);
  if (std::isnan(C) || !(C > 0.0f)) return fail(QR_ERR_INVALID_ARG, "%s: C must be > 0", fn);
  if (!sums) return fail(QR_ERR_INVALID_ARG, "%s: null sums", fn);
  if (n > 0 && (!logp || !logp_prox || !logp_behav || !adv || !mask || !loss))
    return fail(QR_ERR_INVALID_ARG, "%s: null input or loss", fn);
  if (!aligned(logp, 16) || !aligned(logp_prox, 16) || !aligned(logp_behav, 16) ||
      !aligned(adv, 16) || !aligned(loss, 16) || !aligned(grad, 16) || !aligned(mask, 4) ||
      !aligned(sums, 8))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for the fp32 arrays, 4 for mask)", fn);
  const size_t need = align256((size_t)qr::acr_blocks(n) * 3 * sizeof(double));
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 8)))
    return fail(QR_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
  (void)hipGetLastError();
  return hip_status(qr::launch_acr_tis(logp, logp_prox, logp_behav, adv, mask, n, eps, C, loss,
                                       grad, sums, static_cast<double*>(workspace),
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_mx_quantize(const void* A, int64_t R, int64_t K, int64_t lda, int src_bf16, void* codes,
                   uint8_t* scales, void* stream) {
  const char* fn = "qr_mx_quantize";
  if (R < 0 || K < 0 || R >= kMaxDim || K >= kMaxDim)
    return fail(QR_ERR_INVALID_ARG, "%s: bad size (R=%lld K=%lld)", fn, (long long)R, (long long)K);
  if (K % 32 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (src_bf16 != 0 && src_bf16 != 1) return fail(QR_ERR_INVALID_ARG, "%s: src_bf16 must be 0 or 1", fn);
  if (lda < K) return fail(QR_ERR_INVALID_ARG, "%s: lda=%lld < K=%lld", fn, (long long)lda, (long long)K);
  if (R > 0 && K > 0 && (!A || !codes || !scales)) return fail(QR_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (K > 0 && lda % (src_bf16 ? 8 : 4) != 0)
    return fail(QR_ERR_UNSUPPORTED, "%s: rows must start on 16-byte boundaries", fn);
  if (!aligned(A, 16) || !aligned(codes, 16))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for A, codes)", fn);
  (void)hipGetLastError();
  return hip_status(qr::launch_mx_quant(A, R, K, lda, src_bf16, codes, scales,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_mx_gemm(const void* Xq, const uint8_t* sx, const void* Wq, const uint8_t* sw, int64_t M,
               int64_t N, int64_t K, int out, void* Y, int64_t ldy, void* stream) {
  const char* fn = "qr_mx_gemm";
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(QR_ERR_INVALID_ARG, "%s: bad size", fn);
  if (K % 128 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: K=%lld is not a multiple of 128", fn, (long long)K);
  if (out != QR_OUT_BF16 && out != QR_OUT_RAW) return fail(QR_ERR_INVALID_ARG, "%s: bad out", fn);
  if (N * K >= kMaxCodeBytes || M * K >= kMaxCodeBytes)
    return fail(QR_ERR_UNSUPPORTED, "%s: code matrices must stay below 2^31 - 2^16 bytes", fn);
  if (ldy < N) return fail(QR_ERR_INVALID_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (M > 0 && N > 0 && (!Y || (K > 0 && (!Xq || !sx || !Wq || !sw))))
    return fail(QR_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned(Xq, 16) || !aligned(Wq, 16) || !aligned(sx, 16) || !aligned(sw, 16) || !aligned(Y, 16))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for Xq, Wq, sx, sw, Y)", fn);
  (void)hipGetLastError();
  return hip_status(qr::launch_mx_gemm(Xq, sx, Wq, sw, M, N, K, out == QR_OUT_RAW, Y, ldy,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

namespace {

int check_gemm_io(const char* fn, int64_t M, int64_t N, int64_t K, int out, bool need_sx,
                  const void* sx, const void* Wq, const void* sw, void* Y, int64_t ldy) {
  if (out != QR_OUT_BF16 && out != QR_OUT_RAW)
    return fail(QR_ERR_INVALID_ARG, "%s: unknown output mode %d", fn, out);
  if (ldy < N) return fail(QR_ERR_INVALID_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (M > 0 && N > 0) {
    if (!Y) return fail(QR_ERR_INVALID_ARG, "%s: null Y", fn);
    if (K > 0 && !Wq) return fail(QR_ERR_INVALID_ARG, "%s: null Wq", fn);
    if (out == QR_OUT_BF16 && ((need_sx && !sx) || !sw))
      return fail(QR_ERR_INVALID_ARG, "%s: null scales", fn);
  }
  if (!aligned(Wq, 16) || !aligned(Y, 16) || !aligned(sx, 4) || !aligned(sw, 4))
    return fail(QR_ERR_UNSUPPORTED, "%s: misaligned pointer (16 bytes for Wq, Y)", fn);
  return QR_OK;
}

int check_ws(const char* fn, void* ws, size_t bytes, size_t need) {
  if (need == 0) return QR_OK;
  if (!ws) return fail(QR_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got NULL", fn, need);
  if (!aligned(ws, 256)) return fail(QR_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  if (bytes < need)
    return fail(QR_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", fn, need, bytes);
  return QR_OK;
}

int run_gemm(const char* fn, const qr::GemmPlan& plan, const void* Xq, const float* sx,
             const void* Wq, const float* sw, int64_t M, int64_t N, int64_t K, int qt, int out,
             void* Y, int64_t ldy, void* gemm_ws, hipStream_t hs) {
  qr::GemmArgs a;
  a.Xq = static_cast<const uint8_t*>(Xq);
  a.sx = sx;
  a.Wq = static_cast<const uint8_t*>(Wq);
  a.sw = sw;
  a.M = M; a.N = N; a.K = K;
  a.Y = Y; a.ldy = ldy;
  a.out_raw = out == QR_OUT_RAW;
  a.part = plan.splitk > 1 ? gemm_ws : nullptr;
  return hip_status(qr::launch_gemm(plan, qt, a, hs), fn);
}

}  // namespace

int qr_w8a8_gemm(const void* Xq, const float* scale_x, const void* Wq, const float* scale_w,
                 int64_t M, int64_t N, int64_t K, int qt, int out, void* Y, int64_t ldy,
                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "qr_w8a8_gemm";
  int st = check_shape(fn, M, N, K, qt);
  if (st != QR_OK) return st;
  st = check_gemm_io(fn, M, N, K, out, true, scale_x, Wq, scale_w, Y, ldy);
  if (st != QR_OK) return st;
  if (M > 0 && N > 0 && K > 0 && !Xq) return fail(QR_ERR_INVALID_ARG, "%s: null Xq", fn);
  if (!aligned(Xq, 16)) return fail(QR_ERR_UNSUPPORTED, "%s: misaligned Xq", fn);
  if (N * K >= kMaxCodeBytes || M * K >= kMaxCodeBytes)
    return fail(QR_ERR_UNSUPPORTED, "%s: a code matrix of 2^31 - 2^16 bytes or more", fn);
  if (M == 0 || N == 0) return ok();
  const qr::GemmPlan plan = qr::make_plan(M, N, K, qt, g_force_tile, g_force_splitk, g_force_rows);
  st = check_ws(fn, workspace, workspace_bytes, plan.ws_bytes());
  if (st != QR_OK) return st;
  (void)hipGetLastError();
  return run_gemm(fn, plan, Xq, scale_x, Wq, scale_w, M, N, K, qt, out, Y, ldy, workspace,
                  static_cast<hipStream_t>(stream));
}

int qr_w8a8_gemm_quant(const void* Xq, const float* scale_x, const void* Wq, const float* scale_w,
                       int64_t M, int64_t N, int64_t K, int qt, void* Y, int64_t ldy, int64_t q_col0,
                       int64_t q_cols, float q_act_mult, void* Xq_next, float* scale_x_next,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "qr_w8a8_gemm_quant";
  int st = check_shape(fn, M, N, K, qt);
  if (st != QR_OK) return st;
  st = check_gemm_io(fn, M, N, K, QR_OUT_BF16, true, scale_x, Wq, scale_w, Y, ldy);
  if (st != QR_OK) return st;
  if (M > 0 && N > 0 && K > 0 && !Xq) return fail(QR_ERR_INVALID_ARG, "%s: null Xq", fn);
  if (!aligned(Xq, 16)) return fail(QR_ERR_UNSUPPORTED, "%s: misaligned Xq", fn);
  if (N * K >= kMaxCodeBytes || M * K >= kMaxCodeBytes)
    return fail(QR_ERR_UNSUPPORTED, "%s: a code matrix of 2^31 - 2^16 bytes or more", fn);
  if (q_col0 < 0 || q_cols < 0 || q_col0 + q_cols > N)
    return fail(QR_ERR_INVALID_ARG, "%s: quantized columns [%lld, %lld) outside [0, N=%lld)", fn,
                (long long)q_col0, (long long)(q_col0 + q_cols), (long long)N);
  if (q_cols > 0) {
    if (q_col0 % 16 != 0 || q_cols % 16 != 0)
      return fail(QR_ERR_UNSUPPORTED, "%s: q_col0 and q_cols must be multiples of 16", fn);
    if (!std::isfinite(q_act_mult) || !(q_act_mult > 0.0f))
      return fail(QR_ERR_INVALID_ARG, "%s: q_act_mult must be finite and > 0", fn);
    if (M > 0 && (!Xq_next || !scale_x_next))
      return fail(QR_ERR_INVALID_ARG, "%s: null Xq_next or scale_x_next", fn);
    if (!aligned(Xq_next, 16) || !aligned(scale_x_next, 4))
      return fail(QR_ERR_UNSUPPORTED, "%s: misaligned Xq_next (16 bytes) or scale_x_next", fn);
    if (ldy % 8 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: ldy must be a multiple of 8", fn);
  }
  if (M == 0 || N == 0) return ok();
  const qr::GemmPlan plan = qr::make_plan(M, N, K, qt, g_force_tile, g_force_splitk, g_force_rows);
  st = check_ws(fn, workspace, workspace_bytes, qr::kFuseHeaderBytes + plan.part_bytes);
  if (st != QR_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  qr::GemmArgs a;
  a.Xq = static_cast<const uint8_t*>(Xq);
  a.sx = scale_x;
  a.Wq = static_cast<const uint8_t*>(Wq);
  a.sw = scale_w;
  a.M = M; a.N = N; a.K = K;
  a.Y = Y; a.ldy = ldy;
  a.out_raw = 0;
  a.part = plan.splitk > 1 ? ws + qr::kFuseHeaderBytes : nullptr;
  (void)hipGetLastError();
  const bool want = plan.splitk > 1 || q_cols > 0;
  if (g_fuse == 1 && want && N % 4 == 0 && ldy % 4 == 0 && aligned(Y, 16) &&
      qr::fused_ok(plan, qt, M, N)) {
    qr::FuseArgs fa;
    fa.header = ws;
    fa.part = a.part;
    fa.xq2 = static_cast<uint8_t*>(Xq_next);
    fa.sx2 = scale_x_next;
    fa.qc0 = q_col0;
    fa.qcn = q_cols;
    fa.am2 = q_act_mult;
    return hip_status(qr::launch_gemm_fused(plan, qt, a, fa, hs), fn);
  }
  // Separate launches. A split plan whose output is quantized: the GEMM
  // writes its partial sums and one kernel adds them, applies the epilogue
  // and quantizes the column range. Otherwise the GEMM (with its split-K
  // kernel), then the per-token quantizer. The same results either way.
  if (plan.splitk > 1 && q_cols > 0 && qr::splitk_reduce_quant_ok(N, plan.splitk) &&
      aligned(Y, 16)) {
    st = hip_status(qr::launch_gemm(plan, qt, a, hs, false), fn);
    if (st != QR_OK) return st;
    return hip_status(qr::launch_splitk_reduce_quant(plan.splitk, qt, a.part, M, N, scale_x,
                                                     scale_w, Y, ldy, q_col0, q_cols, q_act_mult,
                                                     Xq_next, scale_x_next, hs),
                      fn);
  }
  st = hip_status(qr::launch_gemm(plan, qt, a, hs), fn);
  if (st != QR_OK || q_cols == 0) return st;
  return hip_status(qr::launch_act_quant(static_cast<const uint16_t*>(Y) + q_col0, M, q_cols, ldy,
                                         q_act_mult, qt, Xq_next, scale_x_next, hs),
                    fn);
}

int qr_linear_fused(const void* X, int64_t ldx, float act_mult, const void* Wq, const float* scale_w,
                    int64_t M, int64_t N, int64_t K, int qt, void* Y, int64_t ldy, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const char* fn = "qr_linear_fused";
  int st = check_shape(fn, M, N, K, qt);
  if (st != QR_OK) return st;
  if (!std::isfinite(act_mult) || !(act_mult > 0.0f))
    return fail(QR_ERR_INVALID_ARG, "%s: act_mult must be finite and > 0", fn);
  if (ldx < K) return fail(QR_ERR_INVALID_ARG, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
  st = check_gemm_io(fn, M, N, K, QR_OUT_BF16, false, nullptr, Wq, scale_w, Y, ldy);
  if (st != QR_OK) return st;
  if (M > 0 && N > 0 && K > 0 && !X) return fail(QR_ERR_INVALID_ARG, "%s: null X", fn);
  if (ldx % 8 != 0) return fail(QR_ERR_UNSUPPORTED, "%s: ldx must be a multiple of 8", fn);
  if (!aligned(X, 16)) return fail(QR_ERR_UNSUPPORTED, "%s: misaligned X", fn);
  if (N * K >= kMaxCodeBytes || M * K >= kMaxCodeBytes)
    return fail(QR_ERR_UNSUPPORTED, "%s: a code matrix of 2^31 - 2^16 bytes or more", fn);
  if (M == 0 || N == 0) return ok();
  const qr::GemmPlan plan = qr::make_plan(M, N, K, qt, g_force_tile, g_force_splitk, g_force_rows);
  const size_t xq_bytes = align256((size_t)M * (size_t)K);
  const size_t sx_bytes = align256((size_t)M * 4);
  const size_t head = plan.part_bytes;
  st = check_ws(fn, workspace, workspace_bytes, head + xq_bytes + sx_bytes);
  if (st != QR_OK) return st;
  if (g_force_tile < 0 && (g_small_m > 0 ? qr::small_m_ok(M, N, K, ldx)
                                          : g_small_m == 0 && qr::small_m_auto(M, N, K, ldx))) {
    (void)hipGetLastError();
    return hip_status(qr::launch_small_m_linear(X, ldx, act_mult, Wq, scale_w, M, N, K, qt, Y, ldy,
                                                qr::small_m_rf(N, g_small_m),
                                                static_cast<hipStream_t>(stream)),
                      fn);
  }
  char* ws = static_cast<char*>(workspace);
  void* gws = ws;
  void* xq = ws + head;
  float* sx = reinterpret_cast<float*>(ws + head + xq_bytes);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  st = hip_status(qr::launch_act_quant(X, M, K, ldx, act_mult, qt, xq, sx, hs), fn);
  if (st != QR_OK) return st;
  return run_gemm(fn, plan, xq, sx, Wq, scale_w, M, N, K, qt, QR_OUT_BF16, Y, ldy, gws, hs);
}

int qr_probe_read(const void* buf, size_t bytes, uint32_t* sink, int64_t sink_words,
                  void* stream) {
  const char* fn = "qr_probe_read";
  if (bytes % 16 != 0) return fail(QR_ERR_INVALID_ARG, "%s: bytes must be a multiple of 16", fn);
  if (bytes > 0 && !buf) return fail(QR_ERR_INVALID_ARG, "%s: null buf", fn);
  if (!aligned(buf, 16)) return fail(QR_ERR_UNSUPPORTED, "%s: buf must be 16-byte aligned", fn);
  if (!sink || sink_words < (int64_t)qr::read_probe_blocks())
    return fail(QR_ERR_INVALID_ARG, "%s: sink of %u words needed", fn, qr::read_probe_blocks());
  (void)hipGetLastError();
  return hip_status(qr::launch_read_probe(buf, (int64_t)(bytes / 16), sink,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_probe_copy_stream(int tile, const void* Wq, int64_t N, int64_t ldw, const void* Xq, int64_t M,
                         int64_t ldx, int64_t K, int rows, int flags, uint32_t* sink, int64_t sink_words,
                         void* stream) {
  const char* fn = "qr_probe_copy_stream";
  int bn = 0, bm = 0;
  if (!qr::copy_stream_probe_tile(tile, bn, bm))
    return fail(QR_ERR_INVALID_ARG, "%s: tile %d is not replayed (4, 8 and 10 are)", fn, tile);
  if (N < 1 || M < 1 || K < 128 || K % 128 != 0)
    return fail(QR_ERR_INVALID_ARG, "%s: N, M >= 1 and K a positive multiple of 128 needed", fn);
  if (rows < 8 || rows > bn || rows % 8 != 0)
    return fail(QR_ERR_INVALID_ARG, "%s: rows must be a multiple of 8 in [8, %d]", fn, bn);
  if (flags < 0 || flags > (QR_PROBE_PANEL | QR_PROBE_NO_BARRIER | QR_PROBE_RESIDENT))
    return fail(QR_ERR_INVALID_ARG, "%s: unknown flags %d", fn, flags);
  if (flags & QR_PROBE_PANEL) ldw = K;  // panels have no row stride
  if (ldw < K || ldx < K || ldw % 16 != 0 || ldx % 16 != 0)
    return fail(QR_ERR_INVALID_ARG, "%s: ldw and ldx must be >= K and multiples of 16", fn);
  if (!Wq || !Xq || !sink) return fail(QR_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int64_t wbytes = (flags & QR_PROBE_PANEL) ? N * K : N * ldw;
  if (wbytes >= kMaxCodeBytes || M * ldx >= kMaxCodeBytes)
    return fail(QR_ERR_UNSUPPORTED, "%s: a code matrix of 2^31 - 2^16 bytes or more", fn);
  const int64_t grid = ((N + rows - 1) / rows) * ((M + bm - 1) / bm);
  if (grid > INT32_MAX) return fail(QR_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (sink_words < grid)
    return fail(QR_ERR_INVALID_ARG, "%s: sink of %lld words needed", fn, (long long)grid);
  (void)hipGetLastError();
  return hip_status(qr::launch_copy_stream_probe(tile, Wq, Xq, N, M, K, ldw, ldx, rows, flags, sink,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int qr_probe_mfma(int qt, int blocks, int iters, uint32_t* sink, uint64_t* ticks, int* wall_khz,
                  void* stream) {
  const char* fn = "qr_probe_mfma";
  if (!valid_qt(qt)) return fail(QR_ERR_INVALID_ARG, "%s: unknown qtype %d", fn, qt);
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24))
    return fail(QR_ERR_INVALID_ARG, "%s: blocks in [1, 65536] and iters in [1, 2^24]", fn);
  if (!sink || !ticks || !wall_khz) return fail(QR_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned(ticks, 8)) return fail(QR_ERR_UNSUPPORTED, "%s: ticks must be 8-byte aligned", fn);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return hip_status(e, fn);
  (void)hipGetLastError();
  return hip_status(qr::launch_mfma_probe(qt, blocks, iters, sink, ticks,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
