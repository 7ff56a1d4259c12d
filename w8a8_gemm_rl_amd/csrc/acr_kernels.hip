// Trainer-side ACR objective with truncated importance sampling, per token
// (QuRL paper notes, "Method > Key designs > ACR"), for gfx950.
//
// One streaming pass: each thread takes four consecutive tokens (16-byte
// loads of the three log-probabilities and the advantage, one 4-byte load of
// the mask), writes the token's loss and its gradient in logp, and the block
// reduces (loss sum, valid tokens, clipped tokens) in float64 into its slot of
// a workspace. A second one-block kernel adds the slots in index order, so
// the sums do not depend on scheduling. Token math is fp32.
#include "qr_internal.h"

namespace qr {
namespace {

constexpr int kTok = 4;     // tokens per thread
constexpr int kNT = 256;    // threads per block
constexpr int kPerBlock = kTok * kNT;

struct TokOut {
  float loss, grad;
  bool valid, clipped;
};

__device__ __forceinline__ TokOut acr_token(float lp, float lx, float lb, float A, bool valid,
                                            float eps, float C) {
  TokOut o{0.0f, 0.0f, valid, false};
  if (!valid) return o;
  const float R = expf(lp - lx);  // pi / pi_prox
  const float r = expf(lx - lb);  // pi_prox / pi_behav
  const float w = fminf(r, C);
  const float hi = (1.0f + eps) / r;
  const float Rc = fminf(fmaxf(R, 1.0f - eps), hi);
  const float u = R * A, c = Rc * A;
  const bool unclipped = u <= c;
  o.loss = -w * (unclipped ? u : c);
  o.grad = unclipped ? -w * u : 0.0f;
  o.clipped = !unclipped;
  return o;
}

__global__ __launch_bounds__(kNT) void acr_tis_kernel(
    const float* __restrict__ logp, const float* __restrict__ lprox,
    const float* __restrict__ lbeh, const float* __restrict__ adv,
    const uint8_t* __restrict__ mask, int64_t n, float eps, float C, float* __restrict__ loss,
    float* __restrict__ grad, double* __restrict__ part) {
  __shared__ double red[3][kNT / 64];
  const int64_t t0 = ((int64_t)blockIdx.x * kNT + threadIdx.x) * kTok;
  double s = 0.0, nv = 0.0, nc = 0.0;
  if (t0 + kTok <= n) {
    const float4 a = *reinterpret_cast<const float4*>(logp + t0);
    const float4 b = *reinterpret_cast<const float4*>(lprox + t0);
    const float4 c = *reinterpret_cast<const float4*>(lbeh + t0);
    const float4 d = *reinterpret_cast<const float4*>(adv + t0);
    const uint32_t mk = *reinterpret_cast<const uint32_t*>(mask + t0);
    const float pa[4] = {a.x, a.y, a.z, a.w}, pb[4] = {b.x, b.y, b.z, b.w};
    const float pc[4] = {c.x, c.y, c.z, c.w}, pd[4] = {d.x, d.y, d.z, d.w};
    float lo[4], gr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const TokOut o = acr_token(pa[e], pb[e], pc[e], pd[e], ((mk >> (8 * e)) & 0xffu) != 0, eps, C);
      lo[e] = o.loss;
      gr[e] = o.grad;
      s += (double)o.loss;
      nv += o.valid ? 1.0 : 0.0;
      nc += o.clipped ? 1.0 : 0.0;
    }
    *reinterpret_cast<float4*>(loss + t0) = make_float4(lo[0], lo[1], lo[2], lo[3]);
    if (grad) *reinterpret_cast<float4*>(grad + t0) = make_float4(gr[0], gr[1], gr[2], gr[3]);
  } else {
    for (int64_t t = t0; t < n; ++t) {
      const TokOut o = acr_token(logp[t], lprox[t], lbeh[t], adv[t], mask[t] != 0, eps, C);
      loss[t] = o.loss;
      if (grad) grad[t] = o.grad;
      s += (double)o.loss;
      nv += o.valid ? 1.0 : 0.0;
      nc += o.clipped ? 1.0 : 0.0;
    }
  }
  // Block sums: lane shuffles, then the four waves through LDS, in fixed order.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    nv += __shfl_xor(nv, o, 64);
    nc += __shfl_xor(nc, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = s;
    red[1][threadIdx.x >> 6] = nv;
    red[2][threadIdx.x >> 6] = nc;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kNT / 64; ++w) v += red[threadIdx.x][w];
    part[3 * (int64_t)blockIdx.x + threadIdx.x] = v;
  }
}

// Adds the per-block slots: out = {loss sum, valid, clipped}. Thread i adds
// slots i, i + kNT, ... in order (eight slots' loads issued together before
// they are added), then the kNT partial sums are combined by a fixed
// pairwise tree (strides kNT/2, ..., 1), so the result is the same bits on
// every run.
__global__ __launch_bounds__(kNT) void acr_sum_kernel(const double* __restrict__ part,
                                                      int64_t blocks, double* __restrict__ out) {
  __shared__ double red[3][kNT];
  constexpr int U = 8;
  double v[3] = {0.0, 0.0, 0.0};
  for (int64_t b0 = threadIdx.x; b0 < blocks; b0 += (int64_t)U * kNT) {
    double w[U][3];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = b0 + (int64_t)u * kNT;
      const int64_t bb = b < blocks ? b : blocks - 1;  // in range; dropped below
      w[u][0] = part[3 * bb];
      w[u][1] = part[3 * bb + 1];
      w[u][2] = part[3 * bb + 2];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b0 + (int64_t)u * kNT < blocks) {
        v[0] += w[u][0];
        v[1] += w[u][1];
        v[2] += w[u][2];
      }
    }
  }
  red[0][threadIdx.x] = v[0];
  red[1][threadIdx.x] = v[1];
  red[2][threadIdx.x] = v[2];
  __syncthreads();
#pragma unroll
  for (int h = kNT / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
      red[0][threadIdx.x] += red[0][threadIdx.x + h];
      red[1][threadIdx.x] += red[1][threadIdx.x + h];
      red[2][threadIdx.x] += red[2][threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x < 3) out[threadIdx.x] = red[threadIdx.x][0];
}

}  // namespace

int64_t acr_blocks(int64_t n) { return (n + kPerBlock - 1) / kPerBlock; }

hipError_t launch_acr_tis(const float* logp, const float* lprox, const float* lbeh,
                          const float* adv, const uint8_t* mask, int64_t n, float eps, float C,
                          float* loss, float* grad, double* sums, double* part, hipStream_t st) {
  const int64_t blocks = acr_blocks(n);
  if (blocks > 0)
    hipLaunchKernelGGL(acr_tis_kernel, dim3((unsigned)blocks), dim3(kNT), 0, st, logp, lprox, lbeh,
                       adv, mask, n, eps, C, loss, grad, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(acr_sum_kernel, dim3(1), dim3(kNT), 0, st, part, blocks, sums);
  return hipGetLastError();
}

}  // namespace qr
