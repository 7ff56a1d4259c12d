// Producers of the quantized linear's input, fused with its per-token
// quantization, for gfx950: a norm with the UAQ-folded gain (and bias), and
// SiLU(gate) x up. Each is one HBM pass: a block reads its token row once into
// registers, reduces the row statistics across the block, and writes the codes
// and the token's scale; the producer's own output never reaches memory.
//
// The UAQ factor s is merged into the norm (QuRL paper notes, "Method > Key
// designs > UAQ"): the caller passes gamma' = gamma*s (beta' = beta*s), so
// the norm-fed linear's activation scale carries no extra factor. The down
// projection's input is produced by SiLU x up, not by a norm, so its scale is
// multiplied by act_mult = s.
//
// Arithmetic (fixed so that codes are reproducible bit for bit):
//   norm   per-row statistic in float64 (sum of squares of the exact bf16
//          values, or mean then squared deviations), r = fl32(1/sqrt(. + eps))
//          rounded once; then fp32 products (and the bias add) in a fixed order.
//   SiLU   a = fl32(g*u / (1 + exp(-g))) evaluated in float64 per element.
// This file is compiled with floating-point contraction off: a fused
// multiply-add would round differently from the stated order.
#include "qr_device.h"
#include "qr_internal.h"

#pragma clang fp contract(off)

namespace qr {
namespace {

constexpr int block_threads(int tpr) { return tpr < 256 ? 256 : tpr; }

// Sum over the TPR threads of a row (TPR = 64: the wave; else the block).
template <int TPR>
__device__ __forceinline__ double row_sum(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if constexpr (TPR > 64) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = red[0];
#pragma unroll
    for (int w = 1; w < TPR / 64; ++w) s += red[w];
    __syncthreads();  // red is reused by the next reduction
    v = s;
  }
  return v;
}

template <int TPR>
__device__ __forceinline__ float row_max(float v, float* red) {
  v = wave_max(v);
  if constexpr (TPR > 64) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < TPR / 64; ++w) m = fmaxf(m, red[w]);
    v = m;
  }
  return v;
}

__device__ __forceinline__ void unpack8(const uint4 v, float* h) {
  h[0] = bf16_lo(v.x); h[1] = bf16_hi(v.x); h[2] = bf16_lo(v.y); h[3] = bf16_hi(v.y);
  h[4] = bf16_lo(v.z); h[5] = bf16_hi(v.z); h[6] = bf16_lo(v.w); h[7] = bf16_hi(v.w);
}

__device__ __forceinline__ float absmax8(const float* y) {
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[e]));
  return m;
}

// Norm (KIND 0: RMSNorm, 1: LayerNorm) with the folded gain (and bias), then
// per-token quantization of the fp32 result. One row per TPR threads; row
// length <= MAXC * TPR * 8.
template <int QT, int KIND, int TPR, int MAXC, bool BETA>
__global__ __launch_bounds__(block_threads(TPR)) void norm_quant_kernel(
    const uint16_t* __restrict__ H, int64_t M, int64_t K, int64_t ldh,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
    uint8_t* __restrict__ Xq, float* __restrict__ scale_x) {
  constexpr int RPB = block_threads(TPR) / TPR;
  __shared__ double red64[16];
  __shared__ float red[16];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool valid = row < M;
  const int64_t nch = K >> 3;
  const uint4* hr = reinterpret_cast<const uint4*>(H + (valid ? row : 0) * ldh);
  const int niter = (int)((nch + TPR - 1) / TPR);

  uint4 raw[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t c = lt + (int64_t)i * TPR;
    if (i < niter) raw[i] = hr[c < nch ? c : nch - 1];
  }
  auto live = [&](int i) { return valid && i < niter && lt + (int64_t)i * TPR < nch; };

  // Row statistic in float64.
  float mu = 0.0f;
  if constexpr (KIND == 1) {
    double s1 = 0.0;
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
      if (live(i)) {
        float h[8];
        unpack8(raw[i], h);
#pragma unroll
        for (int e = 0; e < 8; ++e) s1 += (double)h[e];
      }
    s1 = row_sum<TPR>(s1, red64);
    mu = (float)(s1 / (double)K);
  }
  double s2 = 0.0;
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
    if (live(i)) {
      float h[8];
      unpack8(raw[i], h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double d = KIND == 1 ? (double)h[e] - (double)mu : (double)h[e];
        s2 += d * d;
      }
    }
  s2 = row_sum<TPR>(s2, red64);
  const float r = (float)(1.0 / sqrt(s2 / (double)K + (double)eps));

  // y = fl32(fl32(d * r) * gamma') [+ beta'], kept in registers.
  float y[MAXC][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (!live(i)) continue;
    const int64_t c = lt + (int64_t)i * TPR;
    float h[8];
    unpack8(raw[i], h);
    const float4 g0 = reinterpret_cast<const float4*>(gamma)[2 * c];
    const float4 g1 = reinterpret_cast<const float4*>(gamma)[2 * c + 1];
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float b[8] = {};
    if constexpr (BETA) {
      const float4 b0 = reinterpret_cast<const float4*>(beta)[2 * c];
      const float4 b1 = reinterpret_cast<const float4*>(beta)[2 * c + 1];
      b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
      b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = KIND == 1 ? h[e] - mu : h[e];
      float v = (d * r) * g[e];
      if constexpr (BETA) v = v + b[e];
      y[i][e] = v;
    }
    amax = fmaxf(amax, absmax8(y[i]));
  }
  amax = row_max<TPR>(amax, red);
  if (!valid) return;

  const float t = amax / qmax<QT>();
  if (lt == 0) scale_x[row] = t;
  uint2* qr_ = reinterpret_cast<uint2*>(Xq + row * K);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (!live(i)) continue;
    const int64_t c = lt + (int64_t)i * TPR;
    uint2 q = make_uint2(0u, 0u);
    if (t != 0.0f) {
      q.x = quant_codes4<QT>(y[i][0], y[i][1], y[i][2], y[i][3], t);
      q.y = quant_codes4<QT>(y[i][4], y[i][5], y[i][6], y[i][7], t);
    }
    qr_[c] = q;
  }
}

// a = fl32(g*u / (1 + exp(-g))) in float64, then per-token quantization with
// scale fl32(t * act_mult).
template <int QT, int TPR, int MAXC>
__global__ __launch_bounds__(block_threads(TPR)) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ U, int64_t M, int64_t N,
    int64_t ldg, int64_t ldu, float act_mult, uint8_t* __restrict__ Xq,
    float* __restrict__ scale_x) {
  constexpr int RPB = block_threads(TPR) / TPR;
  __shared__ float red[16];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool valid = row < M;
  const int64_t nch = N >> 3;
  const uint4* gr = reinterpret_cast<const uint4*>(G + (valid ? row : 0) * ldg);
  const uint4* ur = reinterpret_cast<const uint4*>(U + (valid ? row : 0) * ldu);
  const int niter = (int)((nch + TPR - 1) / TPR);

  uint4 rg[MAXC], ru[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t c = lt + (int64_t)i * TPR;
    if (i < niter) {
      rg[i] = gr[c < nch ? c : nch - 1];
      ru[i] = ur[c < nch ? c : nch - 1];
    }
  }
  auto live = [&](int i) { return valid && i < niter && lt + (int64_t)i * TPR < nch; };

  float a[MAXC][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (!live(i)) continue;
    float g[8], u[8];
    unpack8(rg[i], g);
    unpack8(ru[i], u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double gd = g[e];
      a[i][e] = (float)((gd * (double)u[e]) / (1.0 + exp(-gd)));
    }
    amax = fmaxf(amax, absmax8(a[i]));
  }
  amax = row_max<TPR>(amax, red);
  if (!valid) return;

  const float t = amax / qmax<QT>();
  if (lt == 0) scale_x[row] = t * act_mult;
  uint2* qr_ = reinterpret_cast<uint2*>(Xq + row * N);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (!live(i)) continue;
    const int64_t c = lt + (int64_t)i * TPR;
    uint2 q = make_uint2(0u, 0u);
    if (t != 0.0f) {
      q.x = quant_codes4<QT>(a[i][0], a[i][1], a[i][2], a[i][3], t);
      q.y = quant_codes4<QT>(a[i][4], a[i][5], a[i][6], a[i][7], t);
    }
    qr_[c] = q;
  }
}

inline unsigned grid_for(int64_t rows, int rpb) { return (unsigned)((rows + rpb - 1) / rpb); }

// Blocks per launch at most 2^21; longer row ranges take several launches.
constexpr int64_t kRowBlocks = int64_t(1) << 21;

template <int QT, int KIND, int TPR, int MAXC>
void launch_norm(const uint16_t* h, int64_t m, int64_t K, int64_t ldh, const float* gamma,
                 const float* beta, float eps, uint8_t* q, float* sx, hipStream_t st) {
  constexpr int NT = block_threads(TPR);
  const dim3 g(grid_for(m, NT / TPR)), b(NT);
  if (beta)
    hipLaunchKernelGGL((norm_quant_kernel<QT, KIND, TPR, MAXC, true>), g, b, 0, st, h, m, K, ldh,
                       gamma, beta, eps, q, sx);
  else
    hipLaunchKernelGGL((norm_quant_kernel<QT, KIND, TPR, MAXC, false>), g, b, 0, st, h, m, K, ldh,
                       gamma, beta, eps, q, sx);
}

template <int QT, int KIND>
hipError_t norm_rows(const uint16_t* h, int64_t M, int64_t K, int64_t ldh, const float* gamma,
                     const float* beta, float eps, uint8_t* q, float* sx, hipStream_t st) {
  // Rows up to 2048: one wave each, four per block; longer rows one block
  // each, 2-4 16-byte chunks per thread.
  const int rpb = K <= 2048 ? 4 : 1;
  for (int64_t r0 = 0; r0 < M; r0 += kRowBlocks * rpb) {
    const int64_t m = M - r0 < kRowBlocks * rpb ? M - r0 : kRowBlocks * rpb;
    const uint16_t* hs = h + r0 * ldh;
    uint8_t* qs = q + r0 * K;
    float* ss = sx + r0;
    if (K <= 2048)
      launch_norm<QT, KIND, 64, 4>(hs, m, K, ldh, gamma, beta, eps, qs, ss, st);
    else if (K <= 4096)
      launch_norm<QT, KIND, 256, 2>(hs, m, K, ldh, gamma, beta, eps, qs, ss, st);
    else if (K <= 8192)
      launch_norm<QT, KIND, 512, 2>(hs, m, K, ldh, gamma, beta, eps, qs, ss, st);
    else if (K <= 16384)
      launch_norm<QT, KIND, 1024, 2>(hs, m, K, ldh, gamma, beta, eps, qs, ss, st);
    else
      launch_norm<QT, KIND, 1024, 4>(hs, m, K, ldh, gamma, beta, eps, qs, ss, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int QT, int TPR, int MAXC>
void launch_silu(const uint16_t* g, const uint16_t* u, int64_t m, int64_t N, int64_t ldg,
                 int64_t ldu, float act_mult, uint8_t* q, float* sx, hipStream_t st) {
  constexpr int NT = block_threads(TPR);
  hipLaunchKernelGGL((silu_mul_quant_kernel<QT, TPR, MAXC>), dim3(grid_for(m, NT / TPR)), dim3(NT),
                     0, st, g, u, m, N, ldg, ldu, act_mult, q, sx);
}

template <int QT>
hipError_t silu_rows(const uint16_t* g, const uint16_t* u, int64_t M, int64_t N, int64_t ldg,
                     int64_t ldu, float act_mult, uint8_t* q, float* sx, hipStream_t st) {
  const int rpb = N <= 2048 ? 4 : 1;
  for (int64_t r0 = 0; r0 < M; r0 += kRowBlocks * rpb) {
    const int64_t m = M - r0 < kRowBlocks * rpb ? M - r0 : kRowBlocks * rpb;
    const uint16_t* gs = g + r0 * ldg;
    const uint16_t* us = u + r0 * ldu;
    uint8_t* qs = q + r0 * N;
    float* ss = sx + r0;
    if (N <= 2048)
      launch_silu<QT, 64, 4>(gs, us, m, N, ldg, ldu, act_mult, qs, ss, st);
    else if (N <= 4096)
      launch_silu<QT, 256, 2>(gs, us, m, N, ldg, ldu, act_mult, qs, ss, st);
    else if (N <= 8192)
      launch_silu<QT, 512, 2>(gs, us, m, N, ldg, ldu, act_mult, qs, ss, st);
    else if (N <= 16384)
      launch_silu<QT, 1024, 2>(gs, us, m, N, ldg, ldu, act_mult, qs, ss, st);
    else
      launch_silu<QT, 1024, 4>(gs, us, m, N, ldg, ldu, act_mult, qs, ss, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_norm_quant(const void* H, int64_t M, int64_t K, int64_t ldh, int kind,
                             const float* gamma, const float* beta, float eps, int qt, void* Xq,
                             float* scale_x, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const uint16_t* h = static_cast<const uint16_t*>(H);
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (qt == kQInt8)
    return kind == 0 ? norm_rows<kQInt8, 0>(h, M, K, ldh, gamma, beta, eps, q, scale_x, st)
                     : norm_rows<kQInt8, 1>(h, M, K, ldh, gamma, beta, eps, q, scale_x, st);
  return kind == 0 ? norm_rows<kQFp8, 0>(h, M, K, ldh, gamma, beta, eps, q, scale_x, st)
                   : norm_rows<kQFp8, 1>(h, M, K, ldh, gamma, beta, eps, q, scale_x, st);
}

hipError_t launch_silu_mul_quant(const void* G, const void* U, int64_t M, int64_t N, int64_t ldg,
                                 int64_t ldu, float act_mult, int qt, void* Xq, float* scale_x,
                                 hipStream_t st) {
  if (M == 0) return hipSuccess;
  const uint16_t* g = static_cast<const uint16_t*>(G);
  const uint16_t* u = static_cast<const uint16_t*>(U);
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (qt == kQInt8) return silu_rows<kQInt8>(g, u, M, N, ldg, ldu, act_mult, q, scale_x, st);
  return silu_rows<kQFp8>(g, u, M, N, ldg, ldu, act_mult, q, scale_x, st);
}

}  // namespace qr
