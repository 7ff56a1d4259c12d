// Block-wise FP8 for gfx950: E4M3FN elements with one power-of-two (E8M0)
// scale per 32 consecutive elements of a row, the scaling the CDNA4 matrix
// cores apply natively (v_mfma_scale_f32_16x16x128_f8f6f4 takes one scale
// byte per row and 32-element block of K). The block-wise variant is
// the one the QuRL pages cite ([fugumt] "Related papers": FP8-RL); its block
// size and scale format are not on the pages, and these are the hardware's.
//
//   mx_quant_kernel  one thread per 32-element block: absmax, exponent X (the
//                    smallest with absmax <= 448 * 2^X), the E8M0 byte X + 127,
//                    and the codes of fl32(v * 2^-X).
//   mx_gemm_kernel   weights on the MFMA A operand, tokens on B; operands go
//                    from global memory straight into registers, D K steps
//                    ahead (no LDS), with the lane's scale byte per operand;
//                    output bf16(acc) or the fp32 accumulators.
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWordBuf = 0x00020000;  // raw buffer resource word 3 (gfx9)
constexpr uint32_t kOOB = 0x80000000u;

// Exponent of a block: smallest X with amax <= 448 * 2^X; amax = f 2^e with
// f in [0.5, 1) and 448 = 0.875 2^9. Clamped to the E8M0 range.
__device__ __forceinline__ int mx_exp(float amax) {
  if (amax == 0.0f) return -127;
  int e;
  const float f = frexpf(amax, &e);
  int X = f <= 0.875f ? e - 9 : e - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

__device__ __forceinline__ uint32_t mx_codes4(float a, float b, float c, float d, int nX) {
  auto sc = [nX](float v) { return fminf(fmaxf(ldexpf(v, nX), -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sc(a), sc(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sc(c), sc(d), w, true);
  return (uint32_t)w;
}

template <bool BF16>
__global__ __launch_bounds__(256) void mx_quant_kernel(const void* __restrict__ A, int64_t R,
                                                       int64_t K, int64_t lda,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t nb = K >> 5;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * nb) return;
  const int64_t row = idx / nb, b = idx - row * nb;
  float v[32];
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(A) + row * lda + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = p[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * i + 2 * e] = bf16_lo(w[e]);
        v[8 * i + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(A) + row * lda + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_exp(amax);
  scales[row * nb + b] = (uint8_t)(X + 127);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = mx_codes4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], -X);
  uint4* out = reinterpret_cast<uint4*>(codes + row * K + b * 32);
  out[0] = make_uint4(q[0], q[1], q[2], q[3]);
  out[1] = make_uint4(q[4], q[5], q[6], q[7]);
}

struct MxParams {
  const uint8_t* Xq;
  const uint8_t* sx;  // [M, K/32] E8M0
  const uint8_t* Wq;
  const uint8_t* sw;  // [N, K/32] E8M0
  int64_t M, N, K;
  void* Y;
  int64_t ldy;
  int out_raw;
  int tiles_m;
};

// Four waves; wave w owns weight rows [64 FN tn + 16 FN w, + 16 FN) and all
// 16 FM tokens of the tile. In the 16x16x128 scaled MFMA, lane l (row l % 16,
// group g = l / 16) supplies the K positions [16 g, 16 g + 16) in its first
// 16 bytes and [64 + 16 g, + 16) in its last 16, and the scale of the
// 32-element block g (measured: a block's scale follows the lane group, not
// the lane's data). So each lane loads those two 16-byte pieces of the
// 128-byte K step and passes the scale byte of block g.
template <int FN, int FM, int D>
__global__ __launch_bounds__(256, 1) void mx_gemm_kernel(const MxParams p) {
  constexpr int BN = 64 * FN, BM = 16 * FM;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tn = blockIdx.x / p.tiles_m, tm = blockIdx.x % p.tiles_m;
  const int64_t N = p.N, M = p.M, K = p.K, nb = K >> 5;
  const int nks = (int)(K >> 7);
  const int64_t n0 = (int64_t)tn * BN + 16 * FN * w;
  if (n0 >= N) return;
  const int lrow = lane & 15, g = lane >> 4;

  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Wq, (short)0, (int)(uint32_t)(N * K), kWordBuf);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Xq, (short)0, (int)(uint32_t)(M * K), kWordBuf);
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.sw, (short)0, (int)(uint32_t)(N * nb), kWordBuf);
  const __amdgpu_buffer_rsrc_t rsx =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.sx, (short)0, (int)(uint32_t)(M * nb), kWordBuf);
  uint32_t oa[FN], ob[FM], sa[FN], sb[FM];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int64_t row = n0 + 16 * i + lrow;
    oa[i] = row < N ? (uint32_t)(row * K + 16 * g) : kOOB;
    sa[i] = row < N ? (uint32_t)(row * nb + g) : kOOB;
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t row = (int64_t)tm * BM + 16 * j + lrow;
    ob[j] = row < M ? (uint32_t)(row * K + 16 * g) : kOOB;
    sb[j] = row < M ? (uint32_t)(row * nb + g) : kOOB;
  }

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i ra[D][FN][2], rb[D][FM][2];
  int ea[D][FN], eb[D][FM];
  auto load = [&](int s, int ks) {
    const int so = ks * 128, ss = ks * 4;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      ra[s][i][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)oa[i], so, 0);
      ra[s][i][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(oa[i] + 64), so, 0);
      ea[s][i] = __builtin_amdgcn_raw_buffer_load_b8(rsw, (int)sa[i], ss, 0);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      rb[s][j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)ob[j], so, 0);
      rb[s][j][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(ob[j] + 64), so, 0);
      eb[s][j] = __builtin_amdgcn_raw_buffer_load_b8(rsx, (int)sb[j], ss, 0);
    }
  };
  auto compute = [&](int s) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const v8i av{ra[s][i][0][0], ra[s][i][0][1], ra[s][i][0][2], ra[s][i][0][3],
                     ra[s][i][1][0], ra[s][i][1][1], ra[s][i][1][2], ra[s][i][1][3]};
        const v8i bv{rb[s][j][0][0], rb[s][j][0][1], rb[s][j][0][2], rb[s][j][0][3],
                     rb[s][j][1][0], rb[s][j][1][1], rb[s][j][1][2], rb[s][j][1][3]};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 0, 0, 0,
                                                                     ea[s][i], 0, eb[s][j]);
      }
  };
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < nks) load(s, s);
  for (int it = 0; it < nks; it += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (it + s < nks) {
        compute(s);
        if (it + s + D < nks) load(s, it + s + D);
      }
    }
  }

  // Register r of lane l: weight row 4 (l / 16) + r, token l % 16.
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = (int64_t)tm * BM + 16 * j + lrow;
      const int64_t n = n0 + 16 * i + 4 * g;
      if (m >= M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (n + r >= N) break;
        if (p.out_raw)
          static_cast<float*>(p.Y)[m * p.ldy + n + r] = acc[i][j][r];
        else
          static_cast<uint16_t*>(p.Y)[m * p.ldy + n + r] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
      }
    }
}

template <int FN, int FM, int D>
hipError_t launch_mx(const MxParams& p, hipStream_t st) {
  const int64_t tiles_n = (p.N + 64 * FN - 1) / (64 * FN);
  MxParams q = p;
  q.tiles_m = (int)((p.M + 16 * FM - 1) / (16 * FM));
  hipLaunchKernelGGL((mx_gemm_kernel<FN, FM, D>), dim3((unsigned)(tiles_n * q.tiles_m)), dim3(256),
                     0, st, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quant(const void* A, int64_t R, int64_t K, int64_t lda, int bf16,
                           void* codes, uint8_t* scales, hipStream_t st) {
  const int64_t total = R * (K >> 5);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  uint8_t* q = static_cast<uint8_t*>(codes);
  if (bf16)
    hipLaunchKernelGGL(mx_quant_kernel<true>, dim3(grid), dim3(256), 0, st, A, R, K, lda, q, scales);
  else
    hipLaunchKernelGGL(mx_quant_kernel<false>, dim3(grid), dim3(256), 0, st, A, R, K, lda, q, scales);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const void* Xq, const uint8_t* sx, const void* Wq, const uint8_t* sw,
                          int64_t M, int64_t N, int64_t K, int out_raw, void* Y, int64_t ldy,
                          hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  MxParams p{static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
             M, N, K, Y, ldy, out_raw, 0};
  // Up to 32 tokens: 64 weight rows per block (one 16-row fragment per
  // wave) for a few hundred blocks; above, 128 rows x 64 tokens (measured
  // faster at M = 256 than 64 rows x 128 tokens, whose operands need more
  // registers than leave room for prefetch).
  if (M <= 16) return launch_mx<1, 1, 4>(p, st);
  if (M <= 32) return launch_mx<1, 2, 4>(p, st);
  return launch_mx<2, 4, 2>(p, st);
}

}  // namespace qr
