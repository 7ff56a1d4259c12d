// Absmax row quantizers for gfx950: per-token activations (bf16 in) and
// per-output-channel weights after the UAQ division (fp32 in).
//
// Both are HBM-bound streaming kernels: each row is read once with 16-byte
// loads (kept in registers when it fits), its absmax is reduced across the
// wavefront with lane shuffles (and across the four waves of a 256-thread
// block through LDS when one block owns a row), and the codes are written
// with coalesced 4- or 8-byte stores. Rows longer than the register budget
// are read twice (the second read is served by L2).
//
// Quantization: QuRL paper notes, "Loss / training strategy" (channel-wise
// weights, token-wise activations, INT8 or FP8); UAQ division by s:
// "Method > Key designs > UAQ".
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {
namespace {

// Threads per block: 256 (four rows of one wave each) when TPR == 64, else
// one row per block of TPR threads (256, 512 or 1024).
constexpr int block_threads(int tpr) { return tpr < 256 ? 256 : tpr; }

// Row maximum: across the wave when each wave owns a row (TPR == 64), else
// across the block's TPR / 64 waves through LDS.
template <int TPR>
__device__ __forceinline__ float row_max(float v, float* red) {
  v = wave_max(v);
  if constexpr (TPR > 64) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < TPR / 64; ++w) v = fmaxf(v, red[w]);
  }
  return v;
}

// The rows of one block, one per TPR threads. MAXC 16-byte chunks per
// thread are kept in registers (row length <= MAXC * TPR * 8).
template <int QT, int TPR, int MAXC>
__device__ __forceinline__ void act_quant_rows(const uint16_t* __restrict__ X, int64_t M,
                                               int64_t K, int64_t ldx, float act_mult,
                                               uint8_t* __restrict__ Xq,
                                               float* __restrict__ scale_x, int64_t base,
                                               float* red) {
  const int lt = threadIdx.x % TPR;
  const int64_t row = base + threadIdx.x / TPR;
  const bool valid = row < M;
  const int64_t nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(X + (valid ? row : 0) * ldx);
  const bool fits = nch <= (int64_t)MAXC * TPR;

  uint4 r[MAXC];
  float amax = 0.0f;
  if (valid && nch > 0) {
    if (fits) {
      // The loads of one row are guarded by a block-uniform trip count
      // only: lanes past the row end re-read its last chunk and drop it,
      // so no load sits behind a divergent branch and all are in flight
      // at once.
      const int64_t last = nch - 1;
      const int niter = (int)((nch + TPR - 1) / TPR);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int64_t c = lt + (int64_t)i * TPR;
        if (i < niter) r[i] = xr[c < nch ? c : last];
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int64_t c = lt + (int64_t)i * TPR;
        if (i < niter && c < nch) amax = fmaxf(amax, absmax8_bf16(r[i]));
      }
    } else {
      for (int64_t c = lt; c < nch; c += TPR) amax = fmaxf(amax, absmax8_bf16(xr[c]));
    }
  }
  amax = row_max<TPR>(amax, red);
  if (!valid) return;

  const float t = amax / qmax<QT>();
  if (lt == 0) scale_x[row] = t * act_mult;
  uint2* qr_ = reinterpret_cast<uint2*>(Xq + row * K);
  if (t == 0.0f) {
    for (int64_t c = lt; c < nch; c += TPR) qr_[c] = make_uint2(0u, 0u);
    return;
  }
  if (fits) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int64_t c = lt + (int64_t)i * TPR;
      if (c < nch) qr_[c] = codes8_bf16<QT>(r[i], t);
    }
  } else {
    for (int64_t c = lt; c < nch; c += TPR) qr_[c] = codes8_bf16<QT>(xr[c], t);
  }
}

template <int QT, int TPR, int MAXC>
__global__ __launch_bounds__(block_threads(TPR)) void act_quant_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx, float act_mult,
    uint8_t* __restrict__ Xq, float* __restrict__ scale_x) {
  __shared__ float red[16];
  act_quant_rows<QT, TPR, MAXC>(X, M, K, ldx, act_mult, Xq, scale_x,
                                (int64_t)blockIdx.x * (block_threads(TPR) / TPR), red);
}

// Positions among four code bytes whose value changed: INT8 any byte
// difference; E4M3FN too, except +0 (0x00) against -0 (0x80).
template <int QT>
__device__ __forceinline__ int changed4(uint32_t a, uint32_t b) {
  int n = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = (a >> (8 * e)) & 0xFFu, y = (b >> (8 * e)) & 0xFFu;
    bool d = x != y;
    if constexpr (QT == kQFp8) d = d && !(((x | y) == 0x80u) && ((x & y) == 0u));
    n += d ? 1 : 0;
  }
  return n;
}

// Streamed fp32 parameters: each is read once per quantization, with the
// non-temporal hint (a plain read stream reaches 6.1-6.3 TB/s on MI355X, a
// non-temporal one 7.0 TB/s; the refresh, which also reads and writes the
// codes, gains about 1%).
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Weights: per-row absmax quantization of W' = fl32(W / s) (DIVS), or of W
// itself when it already holds W' (the per-step refresh). Optionally stores
// W' (may alias W: every element is read by the thread that overwrites it,
// before it does). With CNT, the previous contents of Wq are read just
// before they are overwritten and the number of codes of the row whose value
// changed is stored to row_flips[row].
template <int QT, int TPR, int MAXC, bool DIVS, bool CNT>
__device__ __forceinline__ void weight_quant_rows(const float* W, int64_t N, int64_t K,
                                                  int64_t ldw, float s, uint8_t* __restrict__ Wq,
                                                  float* __restrict__ scale_w, float* Wsc,
                                                  uint32_t* row_flips, int64_t base, float* red,
                                                  int* cnt) {
  const int lt = threadIdx.x % TPR;
  const int64_t row = base + threadIdx.x / TPR;
  const bool valid = row < N;
  const int64_t nch = K >> 2;
  const float4* wr = reinterpret_cast<const float4*>(W + (valid ? row : 0) * ldw);
  const bool fits = nch <= (int64_t)MAXC * TPR;
  auto div4 = [&](float4 v) {
    if constexpr (DIVS) {
      v.x = v.x / s; v.y = v.y / s; v.z = v.z / s; v.w = v.w / s;
    }
    return v;
  };

  float4 r[MAXC];
  float amax = 0.0f;
  if (valid && nch > 0) {
    if (fits) {
      // Loads guarded only by a block-uniform trip count (lanes past the
      // row end re-read its last chunk and drop it), so they are in flight
      // together.
      const int64_t last = nch - 1;
      const int niter = (int)((nch + TPR - 1) / TPR);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int64_t c = lt + (int64_t)i * TPR;
        if (i < niter) r[i] = ld_stream(&wr[c < nch ? c : last]);
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int64_t c = lt + (int64_t)i * TPR;
        if (i < niter) {
          const float4 v = div4(r[i]);
          r[i] = v;
          if (c < nch)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
      }
    } else {
      for (int64_t c = lt; c < nch; c += TPR) {
        const float4 v = div4(ld_stream(&wr[c]));
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      }
    }
  }
  amax = row_max<TPR>(amax, red);
  int nflip = 0;
  if (valid) {
    const float t = amax / qmax<QT>();
    if (lt == 0) scale_w[row] = t;
    uint32_t* qr_ = reinterpret_cast<uint32_t*>(Wq + row * K);
    float4* sr = Wsc ? reinterpret_cast<float4*>(Wsc + row * ldw) : nullptr;
    auto emit = [&](int64_t c, float4 v) {
      if (sr) sr[c] = v;
      const uint32_t q = t != 0.0f ? quant_codes4<QT>(v.x, v.y, v.z, v.w, t) : 0u;
      if constexpr (CNT) nflip += changed4<QT>(qr_[c], q);
      qr_[c] = q;
    };
    if (fits) {
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int64_t c = lt + (int64_t)i * TPR;
        if (c < nch) emit(c, r[i]);
      }
    } else {
      for (int64_t c = lt; c < nch; c += TPR) emit(c, div4(wr[c]));
    }
  }
  if constexpr (CNT) {
    // Row sum of the per-lane counts: across the wave with lane shuffles,
    // then (one row per block) across the block's waves through LDS.
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nflip += __shfl_xor(nflip, o, 64);
    if constexpr (TPR > 64) {
      if ((threadIdx.x & 63) == 0) cnt[threadIdx.x >> 6] = nflip;
      __syncthreads();
      nflip = cnt[0];
#pragma unroll
      for (int w = 1; w < TPR / 64; ++w) nflip += cnt[w];
    }
    if (valid && lt == 0) row_flips[row] = (uint32_t)nflip;
  }
}

template <int QT, int TPR, int MAXC, bool DIVS, bool CNT>
__global__ __launch_bounds__(block_threads(TPR)) void weight_quant_kernel(
    const float* W, int64_t N, int64_t K, int64_t ldw, float s, uint8_t* __restrict__ Wq,
    float* __restrict__ scale_w, float* Wsc, uint32_t* row_flips) {
  __shared__ float red[16];
  __shared__ int cnt[16];
  weight_quant_rows<QT, TPR, MAXC, DIVS, CNT>(W, N, K, ldw, s, Wq, scale_w, Wsc, row_flips,
                                              (int64_t)blockIdx.x * (block_threads(TPR) / TPR),
                                              red, cnt);
}

// gamma' = fl32(gamma * s), beta' = fl32(beta * s): the activation-side s of
// UAQ folded into the norm that produces the linear's input.
__global__ __launch_bounds__(256) void fold_norm_kernel(float* gamma, float* beta, int64_t K,
                                                         float s) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < K; i += (int64_t)gridDim.x * 256) {
    if (gamma) gamma[i] = gamma[i] * s;
    if (beta) beta[i] = beta[i] * s;
  }
}

inline unsigned grid_for(int64_t rows, int rpb) { return (unsigned)((rows + rpb - 1) / rpb); }

// Blocks per launch: at most 2^21 (2^31 work-items at 1024 threads, inside
// the 32-bit dispatch grid); longer row ranges are split into several
// launches on the host.
constexpr int64_t kRowBlocks = int64_t(1) << 21;

}  // namespace

template <int QT, int TPR, int MAXC>
void launch_act_kernel(const uint16_t* x, int64_t m, int64_t K, int64_t ldx, float act_mult,
                       uint8_t* q, float* scale_x, hipStream_t st) {
  constexpr int NT = block_threads(TPR);
  hipLaunchKernelGGL((act_quant_kernel<QT, TPR, MAXC>), dim3(grid_for(m, NT / TPR)), dim3(NT), 0,
                     st, x, m, K, ldx, act_mult, q, scale_x);
}

template <int QT>
hipError_t launch_act_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float act_mult,
                           uint8_t* q, float* scale_x, hipStream_t st) {
  // Short rows: one wave per row, four rows per block. Longer rows: one
  // block per row, sized so that each thread holds at most 1-5 16-byte
  // chunks (few registers: high occupancy for a streaming kernel). Measured
  // on the 7B layer at 256 tokens: 512 threads x 1 chunk for the
  // 3584-element rows and 512 x 5 for the 18944-element ones are each
  // ~1% of the layer step faster than 256 x 2 and 1024 x 4; one wave per
  // 3584-element row is 3% slower.
  const int rpb = K <= 2048 ? 4 : 1;
  for (int64_t r0 = 0; r0 < M; r0 += kRowBlocks * rpb) {
    const int64_t m = M - r0 < kRowBlocks * rpb ? M - r0 : kRowBlocks * rpb;
    const uint16_t* xs = x + r0 * ldx;
    uint8_t* qs = q + r0 * K;
    float* ss = scale_x + r0;
    if (K <= 2048)
      launch_act_kernel<QT, 64, 4>(xs, m, K, ldx, act_mult, qs, ss, st);
    else if (K <= 4096)
      launch_act_kernel<QT, 512, 1>(xs, m, K, ldx, act_mult, qs, ss, st);
    else if (K <= 8192)
      launch_act_kernel<QT, 256, 4>(xs, m, K, ldx, act_mult, qs, ss, st);
    else if (K <= 16384)
      launch_act_kernel<QT, 512, 4>(xs, m, K, ldx, act_mult, qs, ss, st);
    else if (K <= 20480)
      launch_act_kernel<QT, 512, 5>(xs, m, K, ldx, act_mult, qs, ss, st);
    else
      launch_act_kernel<QT, 1024, 4>(xs, m, K, ldx, act_mult, qs, ss, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_act_quant(const void* X, int64_t M, int64_t K, int64_t ldx, float act_mult,
                            int qt, void* Xq, float* scale_x, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (qt == kQInt8) return launch_act_rows<kQInt8>(x, M, K, ldx, act_mult, q, scale_x, st);
  return launch_act_rows<kQFp8>(x, M, K, ldx, act_mult, q, scale_x, st);
}

// Register budget per thread sized to the row (occupancy falls with the
// registers a kernel reserves, and a streaming kernel needs every wave it can
// get): short rows one wave each, four rows per block; longer rows one block
// each, with the fewest 16-byte chunks per thread that hold the row. Rows
// longer than 32768 elements are read twice.
template <int QT, int TPR, int MAXC, bool DIVS, bool CNT>
void launch_weight_kernel(const float* W, int64_t n, int64_t K, int64_t ldw, float s, uint8_t* q,
                          float* scale_w, float* Wsc, uint32_t* flips, hipStream_t st) {
  constexpr int NT = block_threads(TPR);
  hipLaunchKernelGGL((weight_quant_kernel<QT, TPR, MAXC, DIVS, CNT>), dim3(grid_for(n, NT / TPR)),
                     dim3(NT), 0, st, W, n, K, ldw, s, q, scale_w, Wsc, flips);
}

template <int QT, bool DIVS, bool CNT>
hipError_t launch_weight_rows(const float* W, int64_t N, int64_t K, int64_t ldw, float s,
                              uint8_t* q, float* scale_w, float* Wsc, uint32_t* flips,
                              hipStream_t st) {
  // Short rows: one wave per row, four rows per block. Longer rows: one
  // block per row, sized so that each thread holds 4-8 16-byte chunks
  // (measured on MI355X: 256 threads x 4 chunks for 3584-element rows and
  // 1024 x 5 for 18944 beat fewer threads with more chunks each, which cost
  // registers and so waves in flight).
  const int rpb = K <= 1024 ? 4 : 1;
  for (int64_t r0 = 0; r0 < N; r0 += kRowBlocks * rpb) {
    const int64_t n = N - r0 < kRowBlocks * rpb ? N - r0 : kRowBlocks * rpb;
    const float* ws = W + r0 * ldw;
    uint8_t* qs = q + r0 * K;
    float* ss = scale_w + r0;
    float* wsc = Wsc ? Wsc + r0 * ldw : nullptr;
    uint32_t* fs = flips ? flips + r0 : nullptr;
    if (K <= 1024)
      launch_weight_kernel<QT, 64, 4, DIVS, CNT>(ws, n, K, ldw, s, qs, ss, wsc, fs, st);
    else if (K <= 4096)
      launch_weight_kernel<QT, 256, 4, DIVS, CNT>(ws, n, K, ldw, s, qs, ss, wsc, fs, st);
    else if (K <= 8192)
      launch_weight_kernel<QT, 512, 4, DIVS, CNT>(ws, n, K, ldw, s, qs, ss, wsc, fs, st);
    else if (K <= 20480)
      launch_weight_kernel<QT, 1024, 5, DIVS, CNT>(ws, n, K, ldw, s, qs, ss, wsc, fs, st);
    else
      launch_weight_kernel<QT, 1024, 8, DIVS, CNT>(ws, n, K, ldw, s, qs, ss, wsc, fs, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_weight_quant(const float* W, int64_t N, int64_t K, int64_t ldw, float s, int qt,
                               void* Wq, float* scale_w, float* Wsc, hipStream_t st) {
  if (N == 0) return hipSuccess;
  uint8_t* q = static_cast<uint8_t*>(Wq);
  if (qt == kQInt8)
    return launch_weight_rows<kQInt8, true, false>(W, N, K, ldw, s, q, scale_w, Wsc, nullptr, st);
  return launch_weight_rows<kQFp8, true, false>(W, N, K, ldw, s, q, scale_w, Wsc, nullptr, st);
}

hipError_t launch_requant(const float* Wp, int64_t N, int64_t K, int64_t ldw, int qt, void* Wq,
                          float* scale_w, uint32_t* row_flips, hipStream_t st) {
  if (N == 0) return hipSuccess;
  uint8_t* q = static_cast<uint8_t*>(Wq);
  if (qt == kQInt8)
    return row_flips ? launch_weight_rows<kQInt8, false, true>(Wp, N, K, ldw, 1.0f, q, scale_w,
                                                               nullptr, row_flips, st)
                     : launch_weight_rows<kQInt8, false, false>(Wp, N, K, ldw, 1.0f, q, scale_w,
                                                                nullptr, nullptr, st);
  return row_flips ? launch_weight_rows<kQFp8, false, true>(Wp, N, K, ldw, 1.0f, q, scale_w,
                                                            nullptr, row_flips, st)
                   : launch_weight_rows<kQFp8, false, false>(Wp, N, K, ldw, 1.0f, q, scale_w,
                                                             nullptr, nullptr, st);
}

hipError_t launch_fold_norm(float* gamma, float* beta, int64_t K, float s, hipStream_t st) {
  if (K == 0 || (!gamma && !beta)) return hipSuccess;
  hipLaunchKernelGGL(fold_norm_kernel, dim3(grid_for(K, 256)), dim3(256), 0, st, gamma, beta, K, s);
  return hipGetLastError();
}

}  // namespace qr
