// W8A8 GEMM for gfx950: Y[m, n] = epilogue(sum_k Xq[m, k] * Wq[n, k]).
//
// The quantized product of the rollout linear (QuRL paper notes, "Method >
// System integration": INT8/FP8 matrix multiplication; "Loss / training
// strategy": channel-wise weight and token-wise activation scales).
//
// Design (MI355X / CDNA4):
//  * Both operands are K-contiguous ("TN"). Weights feed the MFMA A operand
//    (rows i = output channels n), activations feed the B operand (columns
//    j = tokens m). INT8 uses v_mfma_i32_32x32x32_i8 (full rate on gfx950;
//    the 16x16x64 form runs at half rate and is used only for 16-token
//    tiles), exact int32 accumulation. FP8 E4M3FN uses
//    v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4 with unit block scales
//    (E8M0 127 = 2^0), accumulating in fp32.
//  * A block owns a BN x BM macro tile and a contiguous range of K. Both
//    operand tiles go global -> registers -> LDS. Global loads run two K
//    steps ahead of the MFMAs (two register stages), LDS is double-buffered,
//    and one barrier separates K steps. 16-byte LDS chunks are XOR-swizzled
//    by row so the 16-byte fragment reads of the MFMA operands are free of
//    bank conflicts.
//  * Each lane feeds the MFMA a contiguous 16- or 32-byte run of K for its row.
//    The K order inside one instruction is the same for A and B, so any lane
//    placement of K gives the same dot product.
//  * Split K (when there are too few macro tiles for 256 CUs): each block
//    stores its partial sums to the workspace with plain stores; a second
//    kernel adds the splits in order and applies the epilogue. No
//    cross-block synchronization inside a kernel (agent-scope fences flush
//    and invalidate L2 on this chip), and FP8 sums are deterministic.
//  * Block indices are remapped so that consecutive logical tiles (same
//    weight tile, neighbouring token tiles and K splits) run on the same XCD
//    and share its L2 (blocks are dealt to the 8 XCDs round-robin).
//  * Epilogue: y = bf16_rne(fl32(fl32(fl32(acc) * sx[m]) * sw[n])), or the raw
//    accumulators.
#include <type_traits>

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

// Word 3 of a raw buffer resource on gfx9 parts: 32-bit data format, no
// swizzle; with stride 0 the bound check is offset < num_records.
constexpr int kBufWord3 = 0x00020000;

struct KParams {
  const uint8_t* Xq;
  const float* sx;
  const uint8_t* Wq;
  const float* sw;
  int64_t M, N, K;
  void* Y;       // output, or the split-K partial buffer [splitk][M][N]
  int64_t ldy;   // leading dimension of Y (N for partials)
  int out_raw;   // 1: store raw accumulators (always for partials)
  int vec;       // ldy % 4 == 0: four consecutive outputs may be stored as one vector
  int splitk;
  int tiles_n, tiles_m, nks;
};

// XOR swizzle of the 16-byte chunk index inside an LDS row. The LDS serves
// a 128-bit read for 16 lanes at a time (256 bytes, 64 banks), and the MFMA
// fragment reads put 16 consecutive rows at the same logical chunk: with
// 128-byte rows, rows r and r+1 differ in their bank half, and (r >> 1) & 7
// spreads the 8 row pairs over the 8 chunk slots (measured: no conflicts).
template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
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
  constexpr int CPR = BK / 16;      // 16-byte chunks per LDS row
  constexpr int RSTEP = NT / CPR;   // rows between one thread's consecutive chunks
  constexpr int CA = BN * CPR, CB = BM * CPR;
  constexpr int LA = (CA + NT - 1) / NT, LBn = (CB + NT - 1) / NT;
  constexpr int NACC = MF::NACC;
  constexpr int KI = MF::KI, LB = MF::LB;
  constexpr int NKK = BK / KI;
  constexpr int STAGE = (BN + BM) * BK;
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(NT % CPR == 0 && RSTEP % 16 == 0, "load rows keep one swizzle");
  static_assert(WTN % T == 0 && WTM % T == 0, "wave tile");
  static_assert(BK % KI == 0, "BK vs MFMA depth");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  // ---- logical tile of this block (XCD-aware, see the file comment)
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

  acc_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = acc_t{};

  // ---- per-thread load addressing, computed once. Thread tid moves chunk
  // c_ld of rows r_ld + i * RSTEP with buffer loads: a 32-bit per-thread
  // offset plus the K advance as a scalar offset. Reads outside the buffer
  // return zero: rows past N (or M) and chunks past K on a ragged last step
  // point at offset 2^31, beyond any code matrix (each is under 2 GiB).
  const int c_ld = tid % CPR;
  const int r_ld = tid / CPR;
  const bool ktail = (K % BK) != 0;
  constexpr uint32_t kOOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Wq, (short)0, (int)(uint32_t)(N * K), kBufWord3);
  const __amdgpu_buffer_rsrc_t rsx =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Xq, (short)0, (int)(uint32_t)(M * K), kBufWord3);
  uint32_t oa[LA], ob[LBn];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int64_t row = (int64_t)tn * BN + r_ld + i * RSTEP;
    oa[i] = row < N ? (uint32_t)(row * K + c_ld * 16) : kOOB;
  }
#pragma unroll
  for (int i = 0; i < LBn; ++i) {
    const int64_t row = (int64_t)tm * BM + r_ld + i * RSTEP;
    ob[i] = row < M ? (uint32_t)(row * K + c_ld * 16) : kOOB;
  }
  // LDS write offset of chunk 0 (chunk i adds i * RSTEP rows, same swizzle)
  const int wofs = r_ld * BK + ((c_ld ^ swz<BK>(r_ld)) << 4);

  // LDS read offsets of the MFMA fragments: lane row lr of a fragment, whose
  // base row is a multiple of 16, so the swizzle depends on lr only.
  const int lr = lane % T;
  const int lg = (lane / T) * (LB / 16);
  const int sl = swz<BK>(lr);
  const int rbaseA = (wn * WTN + lr) * BK;
  const int rbaseB = BN * BK + (wm * WTM + lr) * BK;
  int xo0[NKK], xo1[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int c0 = kk * (KI / 16) + lg;
    xo0[kk] = (c0 ^ sl) << 4;
    xo1[kk] = ((c0 + 1) ^ sl) << 4;
  }

  uint4 ra[2][LA], rb[2][LBn];

  auto ld16 = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) -> uint4 {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
  };
  auto gload = [&](int ks, uint4* da, uint4* db) {
    const int kb = ks * BK;  // scalar offset
    if (!ktail || ks + 1 < p.nks) {
#pragma unroll
      for (int i = 0; i < LA; ++i)
        if (CA % NT == 0 || tid + i * NT < CA) da[i] = ld16(rsw, oa[i], kb);
#pragma unroll
      for (int i = 0; i < LBn; ++i)
        if (CB % NT == 0 || tid + i * NT < CB) db[i] = ld16(rsx, ob[i], kb);
    } else {
      const bool kin = kb + c_ld * 16 < K;  // ragged last step
#pragma unroll
      for (int i = 0; i < LA; ++i)
        if (CA % NT == 0 || tid + i * NT < CA) da[i] = ld16(rsw, kin ? oa[i] : kOOB, kb);
#pragma unroll
      for (int i = 0; i < LBn; ++i)
        if (CB % NT == 0 || tid + i * NT < CB) db[i] = ld16(rsx, kin ? ob[i] : kOOB, kb);
    }
  };

  auto sstore = [&](int buf, const uint4* da, const uint4* db) {
    uint8_t* A = smem + buf * STAGE + wofs;
    uint8_t* B = smem + buf * STAGE + BN * BK + wofs;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      if (CA % NT == 0 || tid + i * NT < CA)
        *reinterpret_cast<uint4*>(A + i * RSTEP * BK) = da[i];
#pragma unroll
    for (int i = 0; i < LBn; ++i)
      if (CB % NT == 0 || tid + i * NT < CB)
        *reinterpret_cast<uint4*>(B + i * RSTEP * BK) = db[i];
  };

  auto lds_op = [&](const uint8_t* base, int kk) -> op_t {
    const uint4 u0 = *reinterpret_cast<const uint4*>(base + xo0[kk]);
    if constexpr (LB == 16) {
      return op_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w};
    } else {
      const uint4 u1 = *reinterpret_cast<const uint4*>(base + xo1[kk]);
      return op_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                  (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
    }
  };

  auto compute = [&](int buf) {
    const uint8_t* A = smem + buf * STAGE + rbaseA;
    const uint8_t* B = smem + buf * STAGE + rbaseB;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      op_t a[FN], bb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) a[i] = lds_op(A + i * T * BK, kk);
#pragma unroll
      for (int j = 0; j < FM; ++j) bb[j] = lds_op(B + j * T * BK, kk);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::run(a[i], bb[j], acc[i][j]);
    }
  };

  // ---- main loop: data of K step j lives in register stage j & 1. Step it
  // first writes step it+1 (loaded two steps earlier) to the other LDS
  // buffer, refills those registers with the loads of step it+3, and then
  // runs the MFMAs of step it, so the loads are in flight while the matrix
  // cores work. The loop is unrolled by two so every register stage index is
  // a compile-time constant (a runtime index moves the stages to scratch).
  const int nk = ks1 - ks0;
  auto step = [&](int it, auto stage_c) {
    constexpr int s1 = decltype(stage_c)::value;  // == (it + 1) & 1
    if (it + 1 < nk) sstore(s1, ra[s1], rb[s1]);
    if (it + 3 < nk) gload(ks0 + it + 3, ra[s1], rb[s1]);
    compute(s1 ^ 1);
    __syncthreads();
  };
  if (nk > 0) {
    gload(ks0, ra[0], rb[0]);
    if (nk > 1) gload(ks0 + 1, ra[1], rb[1]);
    sstore(0, ra[0], rb[0]);
    if (nk > 2) gload(ks0 + 2, ra[0], rb[0]);
    __syncthreads();
    for (int it = 0; it < nk; it += 2) {
      step(it, std::integral_constant<int, 1>{});
      if (it + 1 < nk) step(it + 1, std::integral_constant<int, 0>{});
    }
  }

  // ---- epilogue. Lane layout of an MFMA result: for T = 16 register r of
  // lane l is (i = 4*(l/16) + r, j = l%16); for T = 32 it is
  // (i = 8*(r/4) + 4*(l/32) + r%4, j = l%32). Four consecutive registers are
  // four consecutive output channels n of one token m. All scale loads are
  // issued together (buffer loads, zero outside the vectors), then the
  // outputs are converted and stored.
  const bool split = p.splitk > 1;
  const bool raw = split || p.out_raw;
  constexpr int NG = NACC / 4;  // groups of four registers per fragment
  const int jj = lane % T;
  int64_t mrow[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) mrow[j] = (int64_t)tm * BM + wm * WTM + j * T + jj;
  auto ncol = [&](int i, int g) -> int64_t {
    const int ii = (T == 16) ? 4 * (lane / 16) : 8 * g + 4 * (lane / 32);
    return (int64_t)tn * BN + wn * WTN + i * T + ii;
  };
  float sxv[FM];
  float swv[FN][NG][4];
  if (!raw) {
    const __amdgpu_buffer_rsrc_t rsx_ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.sx, (short)0, (int)(uint32_t)(M * 4), kBufWord3);
    const __amdgpu_buffer_rsrc_t rsw_ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.sw, (short)0, (int)(uint32_t)(N * 4), kBufWord3);
#pragma unroll
    for (int j = 0; j < FM; ++j)
      sxv[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
          rsx_, mrow[j] < M ? (int)(mrow[j] * 4) : (int)kOOB, 0, 0));
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int64_t n0 = ncol(i, g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          swv[i][g][e] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
              rsw_, n0 + e < N ? (int)((n0 + e) * 4) : (int)kOOB, 0, 0));
      }
  }
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int r = 4 * g;
        const int64_t n0 = ncol(i, g);
        const int64_t m = mrow[j];
        if (m >= M || n0 >= N) continue;
        const bool full4 = p.vec && n0 + 3 < N;
        if (raw) {
          // int32 or fp32 words, 16 bytes when four outputs fit
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (QT == kQInt8) w[e] = (uint32_t)acc[i][j][r + e];
            else w[e] = __float_as_uint(acc[i][j][r + e]);
          }
          uint32_t* y = static_cast<uint32_t*>(p.Y) + (split ? (int64_t)z * M * N : 0) + m * p.ldy + n0;
          if (full4) {
            *reinterpret_cast<uint4*>(y) = make_uint4(w[0], w[1], w[2], w[3]);
          } else {
            for (int e = 0; e < 4 && n0 + e < N; ++e) y[e] = w[e];
          }
        } else {
          uint32_t bb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) bb[e] = epi_bf16((float)acc[i][j][r + e], sxv[j], swv[i][g][e]);
          uint16_t* y = static_cast<uint16_t*>(p.Y) + m * p.ldy + n0;
          if (full4) {
            *reinterpret_cast<uint2*>(y) = make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
          } else {
            for (int e = 0; e < 4 && n0 + e < N; ++e) y[e] = (uint16_t)bb[e];
          }
        }
      }
}

// Split-K second pass: Y[m, n] = epilogue(sum_{z = 0..S-1} part[z][m][n]),
// summed in split order. One thread per four consecutive n of one m.
template <int QT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const uint32_t* __restrict__ part, int S,
                                                            int64_t M, int64_t N,
                                                            const float* __restrict__ sx,
                                                            const float* __restrict__ sw, void* Y,
                                                            int64_t ldy, int out_raw, int vec) {
  const int64_t nq = (N + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * nq) return;
  const int64_t m = idx / nq;
  const int64_t n0 = (idx % nq) * 4;
  const int cnt = (int)((N - n0) < 4 ? (N - n0) : 4);
  const bool v4 = (N % 4 == 0);
  int32_t si[4] = {0, 0, 0, 0};
  float sf[4] = {0.f, 0.f, 0.f, 0.f};
  for (int zz = 0; zz < S; ++zz) {
    const uint32_t* src = part + (int64_t)zz * M * N + m * N + n0;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (v4) {
      const uint4 u = *reinterpret_cast<const uint4*>(src);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      for (int e = 0; e < cnt; ++e) w[e] = src[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (QT == kQInt8) si[e] += (int32_t)w[e];
      else sf[e] += __uint_as_float(w[e]);
    }
  }
  const bool full4 = vec && cnt == 4;
  if (out_raw) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (QT == kQInt8) ? (uint32_t)si[e] : __float_as_uint(sf[e]);
    uint32_t* y = static_cast<uint32_t*>(Y) + m * ldy + n0;
    if (full4) *reinterpret_cast<uint4*>(y) = make_uint4(w[0], w[1], w[2], w[3]);
    else for (int e = 0; e < cnt; ++e) y[e] = w[e];
  } else {
    const float sxm = sx[m];
    uint32_t bb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = (QT == kQInt8) ? (float)si[e] : sf[e];
      bb[e] = e < cnt ? epi_bf16(a, sxm, sw[n0 + e]) : 0u;
    }
    uint16_t* y = static_cast<uint16_t*>(Y) + m * ldy + n0;
    if (full4) *reinterpret_cast<uint2*>(y) = make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
    else for (int e = 0; e < cnt; ++e) y[e] = (uint16_t)bb[e];
  }
}

// ---------------------------------------------------------------------------
// Tile table. Order matters: the planner and the tuning hook refer to tiles
// by index. (T, BN, BM, BK, WN, WM): MFMA edge, macro tile over N and M,
// K bytes per stage, waves along N and M.
// ---------------------------------------------------------------------------
#define QR_TILES(X)                                          \
  X(16, 64, 16, 128, 4, 1)   /* 0: M <= 16, weight streaming */ \
  X(16, 32, 16, 128, 2, 1)   /* 1: M <= 16, narrow          */ \
  X(32, 128, 32, 128, 4, 1)  /* 2: M <= 32                  */ \
  X(32, 64, 64, 128, 2, 2)   /* 3: M <= 64                  */ \
  X(32, 128, 64, 128, 2, 2)  /* 4: M <= 64, wide            */ \
  X(32, 64, 128, 128, 2, 2)  /* 5: M <= 128                 */ \
  X(32, 128, 128, 128, 2, 2) /* 6: M <= 128, wide           */ \
  X(32, 64, 256, 128, 1, 4)  /* 7: M = 256 decode           */ \
  X(32, 128, 256, 128, 2, 2) /* 8: M = 256 decode, wide     */ \
  X(32, 256, 128, 128, 2, 2) /* 9: large M                  */ \
  X(32, 256, 256, 128, 2, 4) /* 10: large M, 8 waves        */

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
  kp.splitk = plan.splitk;
  kp.tiles_n = (int)plan.tiles_n; kp.tiles_m = (int)plan.tiles_m; kp.nks = (int)plan.nks;
  if (plan.splitk > 1) {
    kp.Y = a.part; kp.ldy = a.N; kp.out_raw = 1; kp.vec = (a.N % 4) == 0;
  } else {
    kp.Y = a.Y; kp.ldy = a.ldy; kp.out_raw = a.out_raw; kp.vec = (a.ldy % 4) == 0;
  }
  const unsigned grid = (unsigned)(plan.tiles_n * plan.tiles_m * plan.splitk);
  hipError_t e = hipErrorInvalidValue;
  int idx = 0;
#define QR_CASE(T, BN, BM, BK, WN, WM)                                               \
  if (plan.tile == idx) {                                                             \
    e = qt == kQInt8 ? launch_one<kQInt8, T, BN, BM, BK, WN, WM>(kp, grid, st)       \
                     : launch_one<kQFp8, T, BN, BM, BK, WN, WM>(kp, grid, st);       \
  }                                                                                   \
  ++idx;
  QR_TILES(QR_CASE)
#undef QR_CASE
  if (e != hipSuccess || plan.splitk <= 1) return e;
  const int64_t work = a.M * ((a.N + 3) / 4);
  const unsigned rgrid = (unsigned)((work + 255) / 256);
  const int vec = (a.ldy % 4) == 0;
  if (qt == kQInt8)
    hipLaunchKernelGGL(splitk_reduce_kernel<kQInt8>, dim3(rgrid), dim3(256), 0, st,
                       static_cast<const uint32_t*>(a.part), plan.splitk, a.M, a.N, a.sx, a.sw,
                       a.Y, a.ldy, a.out_raw, vec);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<kQFp8>, dim3(rgrid), dim3(256), 0, st,
                       static_cast<const uint32_t*>(a.part), plan.splitk, a.M, a.N, a.sx, a.sw,
                       a.Y, a.ldy, a.out_raw, vec);
  return hipGetLastError();
}

}  // namespace qr
