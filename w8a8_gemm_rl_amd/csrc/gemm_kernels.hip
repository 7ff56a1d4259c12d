// W8A8 GEMM for gfx950: Y[m, n] = epilogue(sum_k Xq[m, k] * Wq[n, k]).
//
// The quantized product of the rollout linear (QuRL paper notes, "Method >
// System integration": INT8/FP8 matrix multiplication; "Loss / training
// strategy": channel-wise weight and token-wise activation scales).
//
// Design (MI355X / CDNA4):
//  * Both operands are K-contiguous ("TN"). Weights feed the MFMA A operand
//    (rows i = output channels n), activations feed the B operand (columns
//    j = tokens m). INT8 uses v_mfma_i32_{16x16x64,32x32x32}_i8 (exact int32
//    accumulation); FP8 E4M3FN uses v_mfma_scale_f32_{16x16x128,32x32x64}
//    _f8f6f4 with unit block scales (E8M0 127 = 2^0), fp32 accumulation.
//  * A block owns a BN x BM macro tile and a contiguous range of K. Tiles of
//    both operands are staged through LDS, double-buffered, with an XOR
//    swizzle of 16-byte chunks so that the 16-byte fragment reads of the
//    MFMA operands are bank-conflict free. One barrier per K step.
//  * Each lane feeds the MFMA a contiguous 16- or 32-byte run of K for its row.
//    The K order inside one instruction is the same for A and B, so any lane
//    placement of K gives the same dot product.
//  * Decode-sized M is bound by streaming the weights from HBM; when there are
//    too few macro tiles to cover 256 CUs, K is split across blocks. Partial
//    sums go to a workspace; the last block of a tile to arrive (an atomic
//    counter) adds them in split order, which keeps FP8 results
//    deterministic, and resets the counter for the next call.
//  * Block indices are remapped so that consecutive logical tiles (same weight
//    tile, neighbouring token tiles and K splits) land on the same XCD and
//    share its L2.
//  * Epilogue: y = bf16_rne(fl32(fl32(fl32(acc) * sx[m]) * sw[n])), or the raw
//    accumulators.
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int QT, int T>
struct Mfma;

template <>
struct Mfma<kQInt8, 16> {
  using acc_t = v4i;
  using op_t = v4i;
  static constexpr int KI = 64, LB = 16, NACC = 4;
  static __device__ __forceinline__ acc_t run(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<kQInt8, 32> {
  using acc_t = v16i;
  using op_t = v4i;
  static constexpr int KI = 32, LB = 16, NACC = 16;
  static __device__ __forceinline__ acc_t run(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
// Format code 0 selects FP8 E4M3 for both operands; scale byte 127 is 2^0.
template <>
struct Mfma<kQFp8, 16> {
  using acc_t = v4f;
  using op_t = v8i;
  static constexpr int KI = 128, LB = 32, NACC = 4;
  static __device__ __forceinline__ acc_t run(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};
template <>
struct Mfma<kQFp8, 32> {
  using acc_t = v16f;
  using op_t = v8i;
  static constexpr int KI = 64, LB = 32, NACC = 16;
  static __device__ __forceinline__ acc_t run(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

struct KParams {
  const uint8_t* Xq;
  const float* sx;
  const uint8_t* Wq;
  const float* sw;
  int64_t M, N, K;
  void* Y;
  int64_t ldy;
  int out_raw;
  int splitk;
  int tiles_n, tiles_m, nks;
  void* part;
  int* counters;
};

template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 128) return row & 7;
  else return (row >> 1) & 3;
}

// fl32(acc) * sx * sw -> bf16 bits
__device__ __forceinline__ uint32_t epi_bf16(float a, float sx, float sw) {
  const float t = a * sx;
  const float y = t * sw;
  return f32_to_bf16_rne(y);
}

template <int QT, int T, int BN, int BM, int BK, int WN, int WM>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_kernel(const KParams p) {
  using MF = Mfma<QT, T>;
  using acc_t = typename MF::acc_t;
  using op_t = typename MF::op_t;
  constexpr int NT = 64 * WN * WM;
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FN = WTN / T, FM = WTM / T;
  constexpr int CPR = BK / 16;  // 16-byte chunks per LDS row
  constexpr int CA = BN * CPR, CB = BM * CPR;
  constexpr int LA = (CA + NT - 1) / NT, LBn = (CB + NT - 1) / NT;
  constexpr int NACC = MF::NACC;
  constexpr int KI = MF::KI, LB = MF::LB;
  constexpr int STAGE = (BN + BM) * BK;
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(WTN % T == 0 && WTM % T == 0, "wave tile");
  static_assert(BK % KI == 0, "BK vs MFMA depth");
  static_assert((FN * FM * NACC) % 4 == 0, "partials in 16-byte groups");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int s_last;

  // ---- logical tile of this block (XCD-aware: consecutive logical indices
  // on one XCD; blocks are dispatched to the 8 XCDs round-robin).
  const int G = gridDim.x;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  const int z = b % p.splitk;
  const int t2 = b / p.splitk;
  const int tm = t2 % p.tiles_m;
  const int tn = t2 / p.tiles_m;
  const int ks0 = (int)(((int64_t)z * p.nks) / p.splitk);
  const int ks1 = (int)(((int64_t)(z + 1) * p.nks) / p.splitk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wn = wid % WN, wm = wid / WN;

  const int64_t N = p.N, M = p.M, K = p.K;
  const uint8_t* __restrict__ Wq = p.Wq;
  const uint8_t* __restrict__ Xq = p.Xq;

  acc_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = acc_t{};

  uint4 ra[LA], rb[LBn];

  auto gload = [&](int ks) {
    const int64_t kb = (int64_t)ks * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = tid + i * NT;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (CA % NT == 0 || q < CA) {
        const int r = q / CPR, c = q % CPR;
        const int64_t gn = (int64_t)tn * BN + r;
        const int64_t kk = kb + c * 16;
        if (gn < N && kk < K) v = *reinterpret_cast<const uint4*>(Wq + gn * K + kk);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < LBn; ++i) {
      const int q = tid + i * NT;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (CB % NT == 0 || q < CB) {
        const int r = q / CPR, c = q % CPR;
        const int64_t gm = (int64_t)tm * BM + r;
        const int64_t kk = kb + c * 16;
        if (gm < M && kk < K) v = *reinterpret_cast<const uint4*>(Xq + gm * K + kk);
      }
      rb[i] = v;
    }
  };

  auto sstore = [&](int buf) {
    uint8_t* A = smem + buf * STAGE;
    uint8_t* B = A + BN * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = tid + i * NT;
      if (CA % NT == 0 || q < CA) {
        const int r = q / CPR, c = q % CPR;
        *reinterpret_cast<uint4*>(A + r * BK + ((c ^ swz<BK>(r)) << 4)) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < LBn; ++i) {
      const int q = tid + i * NT;
      if (CB % NT == 0 || q < CB) {
        const int r = q / CPR, c = q % CPR;
        *reinterpret_cast<uint4*>(B + r * BK + ((c ^ swz<BK>(r)) << 4)) = rb[i];
      }
    }
  };

  auto lds_op = [&](const uint8_t* base, int row, int chunk0) -> op_t {
    const uint4 u0 = *reinterpret_cast<const uint4*>(base + row * BK + ((chunk0 ^ swz<BK>(row)) << 4));
    if constexpr (LB == 16) {
      return op_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w};
    } else {
      const int c1 = chunk0 + 1;
      const uint4 u1 = *reinterpret_cast<const uint4*>(base + row * BK + ((c1 ^ swz<BK>(row)) << 4));
      return op_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                  (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
    }
  };

  auto compute = [&](int buf) {
    const uint8_t* A = smem + buf * STAGE;
    const uint8_t* B = A + BN * BK;
    const int lr = lane % T;
    const int lg = (lane / T) * (LB / 16);
#pragma unroll
    for (int kk = 0; kk < BK / KI; ++kk) {
      const int c0 = kk * (KI / 16) + lg;
      op_t a[FN], bb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) a[i] = lds_op(A, wn * WTN + i * T + lr, c0);
#pragma unroll
      for (int j = 0; j < FM; ++j) bb[j] = lds_op(B, wm * WTM + j * T + lr, c0);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::run(a[i], bb[j], acc[i][j]);
    }
  };

  const int nk = ks1 - ks0;
  if (nk > 0) {
    gload(ks0);
    sstore(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      if (it + 1 < nk) gload(ks0 + it + 1);
      compute(it & 1);
      if (it + 1 < nk) sstore((it + 1) & 1);
      __syncthreads();
    }
  }

  // ---- split-K: publish partials, the last block of the tile reduces them.
  if (p.splitk > 1) {
    constexpr int NG = FN * FM * NACC / 4;
    const int64_t ntiles = (int64_t)p.tiles_n * p.tiles_m;
    const int64_t tile = (int64_t)tn * p.tiles_m + tm;
    uint4* part = reinterpret_cast<uint4*>(p.part);
    {
      uint4* mine = part + ((int64_t)z * ntiles + tile) * (NG * NT);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int r = 0; r < NACC; r += 4) {
            const int g = (i * FM + j) * (NACC / 4) + r / 4;
            uint4 v;
            v.x = __builtin_bit_cast(uint32_t, acc[i][j][r + 0]);
            v.y = __builtin_bit_cast(uint32_t, acc[i][j][r + 1]);
            v.z = __builtin_bit_cast(uint32_t, acc[i][j][r + 2]);
            v.w = __builtin_bit_cast(uint32_t, acc[i][j][r + 3]);
            mine[g * NT + tid] = v;
          }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(p.counters + tile, 1);
      s_last = (prev == p.splitk - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int r = 0; r < NACC; r += 4) {
          const int g = (i * FM + j) * (NACC / 4) + r / 4;
          acc_t& A = acc[i][j];
          if constexpr (QT == kQInt8) {
            int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
            for (int zz = 0; zz < p.splitk; ++zz) {
              if (zz == z) {
                s0 += A[r]; s1 += A[r + 1]; s2 += A[r + 2]; s3 += A[r + 3];
              } else {
                const uint4 v = part[((int64_t)zz * ntiles + tile) * (NG * NT) + g * NT + tid];
                s0 += (int)v.x; s1 += (int)v.y; s2 += (int)v.z; s3 += (int)v.w;
              }
            }
            A[r] = s0; A[r + 1] = s1; A[r + 2] = s2; A[r + 3] = s3;
          } else {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
            for (int zz = 0; zz < p.splitk; ++zz) {
              float v0, v1, v2, v3;
              if (zz == z) {
                v0 = A[r]; v1 = A[r + 1]; v2 = A[r + 2]; v3 = A[r + 3];
              } else {
                const uint4 v = part[((int64_t)zz * ntiles + tile) * (NG * NT) + g * NT + tid];
                v0 = __uint_as_float(v.x); v1 = __uint_as_float(v.y);
                v2 = __uint_as_float(v.z); v3 = __uint_as_float(v.w);
              }
              s0 += v0; s1 += v1; s2 += v2; s3 += v3;
            }
            A[r] = s0; A[r + 1] = s1; A[r + 2] = s2; A[r + 3] = s3;
          }
        }
    if (tid == 0) p.counters[tile] = 0;
  }

  // ---- epilogue. Lane layout of an MFMA result: for T = 16 register r of
  // lane l is (i = 4*(l/16) + r, j = l%16); for T = 32 it is
  // (i = 8*(r/4) + 4*(l/32) + r%4, j = l%32). Four consecutive registers are
  // four consecutive output channels n of one token m.
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < NACC; r += 4) {
        const int ii = (T == 16) ? 4 * (lane / 16) : 8 * (r / 4) + 4 * (lane / 32);
        const int jj = lane % T;
        const int64_t n0 = (int64_t)tn * BN + wn * WTN + i * T + ii;
        const int64_t m = (int64_t)tm * BM + wm * WTM + j * T + jj;
        if (m >= M || n0 >= N) continue;
        const acc_t& A = acc[i][j];
        float a4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = (float)A[r + e];
        if (p.out_raw) {
          if constexpr (QT == kQInt8) {
            int32_t* y = static_cast<int32_t*>(p.Y) + m * p.ldy + n0;
            if (n0 + 3 < N) {
              *reinterpret_cast<int4*>(y) = make_int4(A[r], A[r + 1], A[r + 2], A[r + 3]);
            } else {
              for (int e = 0; e < 4 && n0 + e < N; ++e) y[e] = A[r + e];
            }
          } else {
            float* y = static_cast<float*>(p.Y) + m * p.ldy + n0;
            if (n0 + 3 < N) {
              *reinterpret_cast<float4*>(y) = make_float4(a4[0], a4[1], a4[2], a4[3]);
            } else {
              for (int e = 0; e < 4 && n0 + e < N; ++e) y[e] = a4[e];
            }
          }
        } else {
          const float sxm = p.sx[m];
          uint16_t* y = static_cast<uint16_t*>(p.Y) + m * p.ldy + n0;
          if (n0 + 3 < N) {
            const float4 sw4 = *reinterpret_cast<const float4*>(p.sw + n0);
            const uint32_t b0 = epi_bf16(a4[0], sxm, sw4.x), b1 = epi_bf16(a4[1], sxm, sw4.y);
            const uint32_t b2 = epi_bf16(a4[2], sxm, sw4.z), b3 = epi_bf16(a4[3], sxm, sw4.w);
            *reinterpret_cast<uint2*>(y) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
          } else {
            for (int e = 0; e < 4 && n0 + e < N; ++e)
              y[e] = (uint16_t)epi_bf16(a4[e], sxm, p.sw[n0 + e]);
          }
        }
      }
}

// ---------------------------------------------------------------------------
// Tile table. Order matters: the planner and the tuning hook refer to tiles
// by index.
// ---------------------------------------------------------------------------
#define QR_TILES(X)                                  \
  X(16, 64, 16, 128, 4, 1)  /* 0: M <= 16 streaming  */ \
  X(16, 128, 32, 128, 4, 1) /* 1: M <= 32            */ \
  X(16, 128, 64, 128, 2, 2) /* 2: M <= 64            */ \
  X(32, 128, 128, 128, 2, 2) /* 3: M <= 128          */ \
  X(32, 128, 256, 128, 2, 2) /* 4: decode M = 256    */ \
  X(32, 256, 128, 128, 2, 2) /* 5: large M           */ \
  X(32, 256, 256, 128, 2, 2) /* 6: large M           */ \
  X(32, 64, 256, 128, 1, 4) /* 7: decode M = 256, narrow */

#define QR_DESC(T, BN, BM, BK, WN, WM) \
  {"t" #T "_n" #BN "_m" #BM "_k" #BK "_w" #WN "x" #WM, T, BN, BM, BK, 64 * WN * WM},
const TileDesc kTiles[] = {QR_TILES(QR_DESC)};
#undef QR_DESC
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int QT, int T, int BN, int BM, int BK, int WN, int WM>
hipError_t launch_one(const KParams& kp, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<QT, T, BN, BM, BK, WN, WM>), dim3(grid), dim3(64 * WN * WM), 0,
                     st, kp);
  return hipGetLastError();
}

}  // namespace

int num_tiles() { return kNumTiles; }
const TileDesc& tile_desc(int tile) { return kTiles[tile]; }

hipError_t launch_gemm(const GemmPlan& plan, int qt, const GemmArgs& a, hipStream_t st) {
  KParams kp;
  kp.Xq = a.Xq; kp.sx = a.sx; kp.Wq = a.Wq; kp.sw = a.sw;
  kp.M = a.M; kp.N = a.N; kp.K = a.K;
  kp.Y = a.Y; kp.ldy = a.ldy; kp.out_raw = a.out_raw;
  kp.splitk = plan.splitk;
  kp.tiles_n = (int)plan.tiles_n; kp.tiles_m = (int)plan.tiles_m; kp.nks = (int)plan.nks;
  kp.part = a.part; kp.counters = a.counters;
  const unsigned grid = (unsigned)(plan.tiles_n * plan.tiles_m * plan.splitk);
  int idx = 0;
#define QR_CASE(T, BN, BM, BK, WN, WM)                                               \
  if (plan.tile == idx) {                                                             \
    return qt == kQInt8 ? launch_one<kQInt8, T, BN, BM, BK, WN, WM>(kp, grid, st)    \
                        : launch_one<kQFp8, T, BN, BM, BK, WN, WM>(kp, grid, st);    \
  }                                                                                   \
  ++idx;
  QR_TILES(QR_CASE)
#undef QR_CASE
  return hipErrorInvalidValue;
}

}  // namespace qr
