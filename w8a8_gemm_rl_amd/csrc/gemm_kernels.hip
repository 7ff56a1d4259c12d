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
//  * A block owns a BN x BM macro tile (of which the first `rn` weight rows
//    are its own) and a contiguous range of K. The operands move global ->
//    LDS with buffer_load ... lds into an S-slot ring (LDS-DMA). 16-byte LDS
//    chunks are XOR-swizzled by row so the 16-byte fragment reads of the
//    MFMA operands are free of bank conflicts. (Linears of one or two tokens
//    whose input has no producer run instead on the one-launch kernel in
//    small_m_kernels.hip.)
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

#include "qr_copy.h"
#include "qr_device.h"
#include "qr_gemm.h"

namespace qr {
namespace {

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
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

// Fused chain epilogue (one launch per linear of a decode chain): the
// split-K sum and the per-token quantization of the output for the next
// linear happen inside the GEMM launch, across blocks, behind grid-wide
// barriers (all blocks of such a launch are resident at once; the host
// checks). Fields are unused by plain launches.
struct FuseParams {
  uint32_t* bar;   // [0] arrivals, [1] generation (advances by 2 per launch), [2] timeout flag
  uint32_t* pmax;  // [2][kFuseMaxM] per-token absmax bits; buffer (gen / 2) & 1 is this launch's
  uint32_t* part;  // split-K partial sums [splitk][M][N]
  uint8_t* xq2;    // [M][qcn] codes of Y[:, qc0 : qc0 + qcn]
  float* sx2;      // [M] their per-token scales
  int64_t qc0, qcn;
  float am2;       // act_mult of the next linear
  int ipw;         // split-K sum items (256 outputs of one token) per wave
  uint16_t* y;     // bf16 output of a split launch (Y itself holds the partial sums there)
  int64_t ldy;
};

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
  int rn;  // weight rows per tile: a multiple of 8, at most the tile's BN
  FuseParams f;
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


// Logical tile of this block. Blocks are dealt to the 8 XCDs round-robin,
// so block b is renumbered to make runs of consecutive logical tiles (the K
// splits of one output tile, then neighbouring token tiles of one weight
// tile) land on one XCD and share its L2.
__device__ __forceinline__ void block_tile(const KParams& p, int& tn, int& tm, int& z, int& ks0,
                                           int& ks1) {
  const int G = gridDim.x;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  z = b % p.splitk;
  const int t2 = b / p.splitk;
  tm = t2 % p.tiles_m;
  tn = t2 / p.tiles_m;
  ks0 = (int)(((int64_t)z * p.nks) / p.splitk);
  ks1 = (int)(((int64_t)(z + 1) * p.nks) / p.splitk);
}

// ---- epilogue. Lane layout of an MFMA result: for T = 16 register r of
// lane l is (i = 4*(l/16) + r, j = l%16); for T = 32 it is
// (i = 8*(r/4) + 4*(l/32) + r%4, j = l%32). Four consecutive registers are
// four consecutive output channels n of one token m. The scales a lane
// needs are loaded before the K loop (buffer loads, zero outside the
// vectors; they complete before any later copy, so the copy waits stay
// correct), so the epilogue does not wait for memory; then the outputs are
// converted and stored.
template <int FN, int FM, int NG>
struct EpiScales {
  float sx[FM];
  float sw[FN][NG][4];
};

template <int T, int BN, int BM, int WN, int WM>
__device__ __forceinline__ int64_t epi_row(const KParams& p, int tm, int wm, int j, int lane) {
  return (int64_t)tm * BM + wm * (BM / WM) + j * T + lane % T;
}
// Local output channel of register group g of fragment i. Rows at or past
// rn belong to the next tile (rn is a multiple of 8, so a group of four
// never straddles it).
template <int T, int BN, int WN>
__device__ __forceinline__ int epi_nloc(int wn, int i, int g, int lane) {
  const int ii = (T == 16) ? 4 * (lane / 16) : 8 * g + 4 * (lane / 32);
  return wn * (BN / WN) + i * T + ii;
}

template <int QT, int T, int BN, int BM, int WN, int WM, int FN, int FM>
__device__ __forceinline__ void load_scales(const KParams& p, int tn, int tm, int wn, int wm,
                                            int lane,
                                            EpiScales<FN, FM, Mfma<QT, T>::NACC / 4>& sc) {
  constexpr int NG = Mfma<QT, T>::NACC / 4;
  constexpr uint32_t kOOB = 0x80000000u;
  if (p.splitk > 1 || p.out_raw) return;
  const int64_t N = p.N, M = p.M;
  const __amdgpu_buffer_rsrc_t rsx_ = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.sx, (short)0, (int)(uint32_t)(M * 4), kBufWord3);
  const __amdgpu_buffer_rsrc_t rsw_ = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.sw, (short)0, (int)(uint32_t)(N * 4), kBufWord3);
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = epi_row<T, BN, BM, WN, WM>(p, tm, wm, j, lane);
    sc.sx[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
        rsx_, m < M ? (int)(m * 4) : (int)kOOB, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int64_t n0 = (int64_t)tn * p.rn + epi_nloc<T, BN, WN>(wn, i, g, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc.sw[i][g][e] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rsw_, n0 + e < N ? (int)((n0 + e) * 4) : (int)kOOB, 0, 0));
    }
}

template <int QT, int T, int BN, int BM, int WN, int WM, typename acc_t, int FN, int FM>
__device__ __forceinline__ void store_tile(const KParams& p, const acc_t (&acc)[FN][FM],
                                           const EpiScales<FN, FM, Mfma<QT, T>::NACC / 4>& sc,
                                           int tn, int tm, int z, int wn, int wm, int lane) {
  constexpr int NACC = Mfma<QT, T>::NACC;
  const int64_t N = p.N, M = p.M;
  const bool split = p.splitk > 1;
  const bool raw = split || p.out_raw;
  constexpr int NG = NACC / 4;  // groups of four registers per fragment
  int64_t mrow[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) mrow[j] = epi_row<T, BN, BM, WN, WM>(p, tm, wm, j, lane);
  auto nloc = [&](int i, int g) -> int { return epi_nloc<T, BN, WN>(wn, i, g, lane); };
  auto ncol = [&](int i, int g) -> int64_t { return (int64_t)tn * p.rn + nloc(i, g); };
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int r = 4 * g;
        const int64_t n0 = ncol(i, g);
        const int64_t m = mrow[j];
        if (m >= M || n0 >= N || nloc(i, g) >= p.rn) continue;
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
          for (int e = 0; e < 4; ++e) bb[e] = epi_bf16((float)acc[i][j][r + e], sc.sx[j], sc.sw[i][g][e]);
          uint16_t* y = static_cast<uint16_t*>(p.Y) + m * p.ldy + n0;
          if (full4) {
            *reinterpret_cast<uint2*>(y) = make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
          } else {
            for (int e = 0; e < 4 && n0 + e < N; ++e) y[e] = (uint16_t)bb[e];
          }
        }
      }
}

// bf16 epilogue staged through LDS: every lane converts its groups of four
// outputs and writes them (8 bytes) to a [CH][LDT] bf16 tile, then the block
// stores the owned rows of each token as 16-byte pieces (the N tail one by
// one); tiles whose tokens do not all fit the LDS go in chunks of CH tokens
// (a multiple of the wave tile's tokens, so each wave writes in one chunk).
// Requires ldy % 8 == 0 and no split (checked by the caller); the tile's
// first output column tn * rn is a multiple of 8 and Y is 16-byte aligned,
// so every full piece is an aligned 16-byte store.
template <int QT, int T, int BN, int BM, int WN, int WM, int LDT, int CH, typename acc_t, int FN,
          int FM>
__device__ __forceinline__ void store_tile_staged(
    const KParams& p, const acc_t (&acc)[FN][FM],
    const EpiScales<FN, FM, Mfma<QT, T>::NACC / 4>& sc, uint8_t* smem, int tn, int tm, int wn,
    int wm, int lane, int tid) {
  constexpr int NG = Mfma<QT, T>::NACC / 4;
  constexpr int NT = 64 * WN * WM;
  constexpr int WTM = BM / WM;
  static_assert((LDT * 2) % 8 == 0, "8-byte aligned staged rows");
  static_assert(CH % WTM == 0 && CH >= WTM && CH <= BM, "chunks of whole wave tiles");
  uint16_t* so = reinterpret_cast<uint16_t*>(smem);
  const int64_t N = p.N, M = p.M;
  const int64_t n0 = (int64_t)tn * p.rn;
  const int own = (int)((N - n0) < p.rn ? (N - n0) : p.rn);  // owned output columns
  const int mv = (int)((M - (int64_t)tm * BM) < BM ? (M - (int64_t)tm * BM) : BM);
  const int cpt = (own + 7) / 8;  // 16-byte pieces per token row
  uint16_t* Y = static_cast<uint16_t*>(p.Y) + ((int64_t)tm * BM) * p.ldy + n0;
#pragma unroll
  for (int c0 = 0; c0 < BM; c0 += CH) {
    __syncthreads();  // the operand ring (first chunk) or the last chunk is no longer read
    if (wm * WTM >= c0 && wm * WTM < c0 + CH) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int ml = wm * WTM + j * T + lane % T - c0;  // token within the chunk
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const int nl = epi_nloc<T, BN, WN>(wn, i, g, lane);
            uint32_t bb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              bb[e] = epi_bf16((float)acc[i][j][4 * g + e], sc.sx[j], sc.sw[i][g][e]);
            *reinterpret_cast<uint2*>(so + ml * LDT + nl) =
                make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
          }
        }
    }
    __syncthreads();
    const int cm = (mv - c0) < CH ? (mv - c0) : CH;  // valid tokens of the chunk
    for (int c = tid; c < cm * cpt; c += NT) {
      const int ml = c / cpt, nl = 8 * (c - (c / cpt) * cpt);
      const uint16_t* src = so + ml * LDT + nl;
      uint16_t* dst = Y + (int64_t)(c0 + ml) * p.ldy + nl;
      if (nl + 8 <= own) {
        // Non-temporal: the tile's outputs leave in one burst at the end of
        // the kernel and are read by another launch, usually from another
        // XCD's L2; streaming them out drains the burst sooner.
        const uint2 lo = *reinterpret_cast<const uint2*>(src);
        const uint2 hi = *reinterpret_cast<const uint2*>(src + 4);
        const v4u_t v = {lo.x, lo.y, hi.x, hi.y};
        __builtin_nontemporal_store(v, reinterpret_cast<v4u_t*>(dst));
      } else {
        for (int e = 0; nl + e < own; ++e) dst[e] = src[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused chain epilogue.
//
// Barrier: bar[0] counts arriving blocks; the last one resets it to zero and
// then publishes the next generation in bar[1], which the others wait for.
// Generations advance by exactly 2 per launch (an intermediate barrier
// publishes g0 + 1, the last g0 + 2), so (g0 / 2) & 1 alternates between
// launches and selects this launch's half of the per-token absmax buffer;
// the launch clears the other half for the next one. Both words and both
// halves start at zero (the caller zeroes the workspace header once) and
// every completed launch leaves them so.
//
// The blocks of one launch run on different XCDs, whose L2 caches are not
// kept coherent with each other for ordinary stores. Every word one block
// writes and another reads inside the launch (barrier words, per-token
// maxima, split-K partial sums) is therefore stored, loaded or updated with
// device-scope atomic operations, which the hardware performs at the
// device's point of coherence; a wave waits for its own such operations
// (vmcnt 0) before its block arrives. No cache-wide write-back or
// invalidate is issued (one per wave cost about 0.2 us each, serialized per
// XCD). Ordinary stores (bf16 outputs, codes, the next launch's cleared
// half) are only read by later launches.
// The wait is bounded: a block that waits for more than about 0.3 s sets
// bar[2] and goes on (results are then wrong but the kernel ends).
// ---------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_own_memory_ops() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Read by every wave (one load each, no LDS: some tiles use all of it). It
// cannot change before this block has arrived at the first barrier.
__device__ __forceinline__ uint32_t fuse_generation(uint32_t* bar) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)ld_dev(&bar[1]));
}

__device__ __forceinline__ void grid_barrier(uint32_t* bar, uint32_t target) {
  wait_own_memory_ops();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == gridDim.x) {
      st_dev(&bar[0], 0u);
      wait_own_memory_ops();  // the reset lands before any block can arrive again
      st_dev(&bar[1], target);
    } else {
      int spins = 0;
      while (ld_dev(&bar[1]) != target) {
        if (++spins > kSpinLimit) {
          __hip_atomic_fetch_or(&bar[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  __syncthreads();
}

// Split-K partial sums of the fused path, with device-scope stores (another
// block adds them after the barrier). N % 4 == 0 there, so every group of
// four outputs is 16 contiguous, 16-byte aligned bytes.
template <int QT, int T, int BN, int BM, int WN, int WM, typename acc_t, int FN, int FM>
__device__ __forceinline__ void store_partials_dev(const KParams& p, const acc_t (&acc)[FN][FM],
                                                   int tn, int tm, int z, int wn, int wm,
                                                   int lane) {
  constexpr int NG = Mfma<QT, T>::NACC / 4;
  const int64_t N = p.N, M = p.M;
  uint32_t* part = p.f.part + (int64_t)z * M * N;
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int nl = epi_nloc<T, BN, WN>(wn, i, g, lane);
        const int64_t n0 = (int64_t)tn * p.rn + nl;
        const int64_t m = epi_row<T, BN, BM, WN, WM>(p, tm, wm, j, lane);
        if (m >= M || n0 >= N || nl >= p.rn) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (QT == kQInt8) w[e] = (uint32_t)acc[i][j][4 * g + e];
          else w[e] = __float_as_uint(acc[i][j][4 * g + e]);
        }
        uint64_t* y = reinterpret_cast<uint64_t*>(part + m * N + n0);
        st_dev64(y, (uint64_t)w[0] | ((uint64_t)w[1] << 32));
        st_dev64(y + 1, (uint64_t)w[2] | ((uint64_t)w[3] << 32));
      }
}

__device__ __forceinline__ uint32_t* pmax_half(const FuseParams& f, uint32_t g0, int which) {
  return f.pmax + (int64_t)(((g0 >> 1) + which) & 1) * qr::kFuseMaxM;
}

// Clear the other half of the absmax buffer for the next launch.
__device__ __forceinline__ void clear_next_pmax(const FuseParams& f, uint32_t g0) {
  uint32_t* nx = pmax_half(f, g0, 1);
  const int nt = blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * nt + threadIdx.x; i < qr::kFuseMaxM;
       i += (int64_t)gridDim.x * nt)
    st_dev(&nx[i], 0u);
}

// |bf16| of the two halves of a packed word, as fp32
__device__ __forceinline__ float absmax2(uint32_t w) {
  return fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w)));
}

// Codes of four bf16 outputs (packed in two words) with step t; zero step:
// zero codes (an all-zero quantized row), as the per-token quantizer.
template <int QT>
__device__ __forceinline__ uint32_t codes4_of(uint32_t w0, uint32_t w1, float t) {
  if (t == 0.0f) return 0u;
  return quant_codes4<QT>(bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1), t);
}

// No split: the outputs are still in the accumulators. Per-token absmax of
// the quantized columns (lanes, then the waves that share the tokens through
// LDS, then one atomic max per token and block), the bf16 stores, the
// barrier, then the codes from the same bf16 values.
template <int QT, int T, int BN, int BM, int WN, int WM, int LDT, int CH, typename acc_t, int FN,
          int FM>
__device__ __forceinline__ void fused_direct_tail(const KParams& p, const acc_t (&acc)[FN][FM],
                                                  const EpiScales<FN, FM, Mfma<QT, T>::NACC / 4>& sc,
                                                  uint8_t* smem, uint32_t g0, int tn, int tm, int wn,
                                                  int wm, int lane, int tid) {
  constexpr int NG = Mfma<QT, T>::NACC / 4;
  constexpr int WTM = BM / WM;
  const FuseParams& f = p.f;
  const int64_t N = p.N, M = p.M;
  const int64_t q0 = f.qc0, q1 = f.qc0 + f.qcn;
  auto nloc = [&](int i, int g) -> int { return epi_nloc<T, BN, WN>(wn, i, g, lane); };
  auto inq = [&](int i, int g) -> bool {
    const int64_t n0 = (int64_t)tn * p.rn + nloc(i, g);
    return nloc(i, g) < p.rn && n0 < N && n0 >= q0 && n0 < q1;
  };
  auto ybits = [&](int i, int j, int g, int e) -> uint32_t {
    return epi_bf16((float)acc[i][j][4 * g + e], sc.sx[j], sc.sw[i][g][e]);
  };
  // ---- per-token absmax of this block's quantized columns
  float tmx[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        if (inq(i, g)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v = fmaxf(v, fabsf(__uint_as_float(ybits(i, j, g, e) << 16)));
        }
    // lanes holding the same token: l % T
#pragma unroll
    for (int o = T; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    tmx[j] = v;
  }
  uint32_t* red = reinterpret_cast<uint32_t*>(smem);  // [BM] token maxima (bits)
  __syncthreads();  // every wave is past its last read of the operand ring
  for (int t = tid; t < BM; t += 64 * WN * WM) red[t] = 0u;
  __syncthreads();
  if (lane < T) {
#pragma unroll
    for (int j = 0; j < FM; ++j) atomicMax(&red[wm * WTM + j * T + lane], __float_as_uint(tmx[j]));
  }
  __syncthreads();
  const int64_t bn0 = (int64_t)tn * p.rn;
  const int64_t bn1 = bn0 + p.rn < N ? bn0 + p.rn : N;
  const bool any_q = bn0 < q1 && bn1 > q0;  // this block owns quantized columns
  uint32_t* pm = pmax_half(f, g0, 0);
  if (any_q) {
    for (int t = tid; t < BM; t += 64 * WN * WM) {
      const int64_t m = (int64_t)tm * BM + t;
      if (m < M) atomicMax(&pm[m], red[t]);
    }
  }
  // ---- bf16 outputs
  if (CH >= WTM && (p.ldy & 7) == 0)
    store_tile_staged<QT, T, BN, BM, WN, WM, LDT, (CH >= WTM ? CH : WTM)>(p, acc, sc, smem, tn, tm,
                                                                           wn, wm, lane, tid);
  else
    store_tile<QT, T, BN, BM, WN, WM>(p, acc, sc, tn, tm, 0, wn, wm, lane);
  clear_next_pmax(f, g0);
  grid_barrier(f.bar, g0 + 2);
  if (!any_q) return;
  // ---- codes of the quantized columns, from the same bf16 values
  const float Q = qmax<QT>();
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = epi_row<T, BN, BM, WN, WM>(p, tm, wm, j, lane);
    if (m >= M) continue;
    const float t = __uint_as_float(ld_dev(&pm[m])) / Q;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (!inq(i, g)) continue;
        const int64_t n0 = bn0 + nloc(i, g);
        const uint32_t w0 = ybits(i, j, g, 0) | (ybits(i, j, g, 1) << 16);
        const uint32_t w1 = ybits(i, j, g, 2) | (ybits(i, j, g, 3) << 16);
        *reinterpret_cast<uint32_t*>(f.xq2 + m * f.qcn + (n0 - q0)) = codes4_of<QT>(w0, w1, t);
      }
  }
  // the scales, by the block that owns the first quantized column
  if (bn0 <= q0 && q0 < bn1) {
    for (int t = tid; t < BM; t += 64 * WN * WM) {
      const int64_t m = (int64_t)tm * BM + t;
      if (m < M) f.sx2[m] = (__uint_as_float(ld_dev(&pm[m])) / Q) * f.am2;
    }
  }
}

// Split K: the partial sums are in the workspace. After the first barrier
// every wave adds up to f.ipw items of 256 outputs of one token (in split
// order, as the separate reduction kernel does), stores their bf16 values,
// and keeps them in registers for the codes; per-token absmax by one atomic
// max per item; second barrier; codes.
template <int QT, int NW>
__device__ __forceinline__ void fused_splitk_tail(const KParams& p, uint32_t g0, int wid, int lane) {
  constexpr int kItems = kFuseItems;
  const FuseParams& f = p.f;
  const int64_t N = p.N, M = p.M;
  const int S = p.splitk;
  const bool quant = f.qcn > 0;
  const int64_t q0 = f.qc0, q1 = f.qc0 + f.qcn;
  grid_barrier(f.bar, quant ? g0 + 1 : g0 + 2);
  const int64_t nseg = (N + 255) / 256;
  const int64_t items = M * nseg;
  const int64_t tw = (int64_t)gridDim.x * NW;
  const int64_t gw = (int64_t)blockIdx.x * NW + wid;
  uint32_t* pm = pmax_half(f, g0, 0);
  uint32_t keep[kItems][2];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    keep[r][0] = keep[r][1] = 0u;
    const int64_t it = gw + r * tw;
    if (r >= f.ipw || it >= items) continue;
    const int64_t m = it / nseg;
    const int64_t n0 = (it - m * nseg) * 256 + 4 * lane;
    float amax = 0.0f;
    if (n0 < N) {
      const uint32_t* src = f.part + m * N + n0;
      int32_t si[4] = {0, 0, 0, 0};
      float sf[4] = {0.f, 0.f, 0.f, 0.f};
      uint4 w[8];
#pragma unroll
      for (int zz = 0; zz < 8; ++zz)
        if (zz < S) {
          const uint64_t* q = reinterpret_cast<const uint64_t*>(src + (int64_t)zz * M * N);
          const uint64_t lo = ld_dev64(q), hi = ld_dev64(q + 1);
          w[zz] = make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
        }
#pragma unroll
      for (int zz = 0; zz < 8; ++zz) {
        if (zz < S) {
          const uint32_t u[4] = {w[zz].x, w[zz].y, w[zz].z, w[zz].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (QT == kQInt8) si[e] += (int32_t)u[e];
            else sf[e] += __uint_as_float(u[e]);
          }
        }
      }
      const float sxm = p.sx[m];
      uint32_t bb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = (QT == kQInt8) ? (float)si[e] : sf[e];
        bb[e] = epi_bf16(a, sxm, p.sw[n0 + e]);
      }
      keep[r][0] = bb[0] | (bb[1] << 16);
      keep[r][1] = bb[2] | (bb[3] << 16);
      *reinterpret_cast<uint2*>(f.y + m * f.ldy + n0) = make_uint2(keep[r][0], keep[r][1]);
      if (quant && n0 >= q0 && n0 < q1) amax = fmaxf(absmax2(keep[r][0]), absmax2(keep[r][1]));
    }
    if (quant) {
      amax = wave_max(amax);
      if (lane == 0) atomicMax(&pm[m], __float_as_uint(amax));
    }
  }
  clear_next_pmax(f, g0);
  if (!quant) return;
  grid_barrier(f.bar, g0 + 2);
  const float Q = qmax<QT>();
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int64_t it = gw + r * tw;
    if (r >= f.ipw || it >= items) continue;
    const int64_t m = it / nseg;
    const int64_t n0 = (it - m * nseg) * 256 + 4 * lane;
    if (n0 >= N || n0 < q0 || n0 >= q1) continue;
    const float t = __uint_as_float(ld_dev(&pm[m])) / Q;
    *reinterpret_cast<uint32_t*>(f.xq2 + m * f.qcn + (n0 - q0)) = codes4_of<QT>(keep[r][0], keep[r][1], t);
    if (n0 == q0) f.sx2[m] = t * f.am2;
  }
}

// ---------------------------------------------------------------------------
// LDS-DMA GEMM. Operand tiles move from global memory straight into an
// S-slot LDS ring with the copies of qr_copy.h; S - 1 K steps are in flight.
// Each wave waits for its own copies with an explicit vmcnt and one barrier
// per K step publishes them (and frees the slot the next copies overwrite).
// The copies of step it + S - 1 are issued in groups between the MFMA
// sub-steps of step it, so their issue overlaps the matrix work. The
// swizzle is applied on the global side: the lane that owns physical chunk
// c of LDS row r fetches logical chunk c ^ swz(r).
// ---------------------------------------------------------------------------
template <int QT, int T, int BN, int BM, int WN, int WM, int S, int BK, bool NTW, bool FUSE>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_dma_kernel(const KParams p) {
  using MF = Mfma<QT, T>;
  using acc_t = typename MF::acc_t;
  using op_t = typename MF::op_t;
  static_assert(BK == 128 || BK == 64, "K step of 64 or 128 bytes");
  constexpr int RB = 1024 / BK;  // rows per 1 KB copy
  constexpr int CPR = BK / 16;   // 16-byte chunks per row
  constexpr int NW = WN * WM;
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FN = WTN / T, FM = WTM / T;
  constexpr int KI = MF::KI, LB = MF::LB;
  constexpr int NKK = BK / KI;
  static_assert(NKK >= 1, "an MFMA's K fits the step");
  // 1 KB row blocks (RB rows of BK bytes) per stage; the token part is
  // padded so every wave issues the same number of copies.
  constexpr int IA = BN / RB;
  constexpr int IB0 = BM / RB;
  constexpr int IB = IB0 + (NW - IB0 % NW) % NW;
  constexpr int NA = IA / NW, NB = IB / NW, NI = NA + NB;
  constexpr int GA = (NA + 3) / 4, GB = (NB + 3) / 4, NG = GA + GB;  // M0 groups
  constexpr int STAGE = (IA + IB) * 1024;
  static_assert(BN % RB == 0 && BM % RB == 0 && IA % NW == 0, "row blocks per wave");
  static_assert(WTN % T == 0 && WTM % T == 0, "wave tile");
  static_assert(S >= 2 && S <= 8 && (S - 2) * NI <= 63, "ring depth");
  static_assert(S * STAGE <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  int tn, tm, z, ks0, ks1;
  block_tile(p, tn, tm, z, ks0, ks1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wid % WN, wm = wid / WN;
  const int64_t N = p.N, M = p.M, K = p.K;

  acc_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = acc_t{};

  // ---- copy addressing. Wave wid moves weight row blocks wid*NA + i and
  // token row blocks wid*NB + i. Lane l covers row RB*rb + l/CPR of the
  // block, physical chunk l%CPR. Rows past the tile (rn), past N or M, or in the
  // padded token rows point at offset 2^31 (beyond any code matrix, which is
  // kept below 2^31 - 2^16 bytes so the bias below stays out of range) and
  // read as zero. Offsets are biased by -1 KB * (i % 4), the instruction
  // offset of copy i within its M0 group.
  constexpr uint32_t kOOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Wq, (short)0, (int)(uint32_t)(N * K), kBufWord3);
  const __amdgpu_buffer_rsrc_t rsx =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Xq, (short)0, (int)(uint32_t)(M * K), kBufWord3);
  const int lrow = lane / CPR, pch = lane % CPR;
  uint32_t oa[NA], ob[NB];
  bool ka[NA], kb[NB];  // copy i holds real K bytes on the ragged last step
  const bool ktail = (K % BK) != 0;
  const int krem = (int)(K % BK);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = (wid * NA + i) * RB + lrow;
    const int c = pch ^ swz<BK>(r);
    const int64_t row = (int64_t)tn * p.rn + r;
    const uint32_t bias = 1024u * (uint32_t)(i % 4);
    ka[i] = c * 16 < krem;
    oa[i] = ((r < p.rn && row < N) ? (uint32_t)(row * K + c * 16) : kOOB) - bias;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = (wid * NB + i) * RB + lrow;
    const int c = pch ^ swz<BK>(r);
    const int64_t row = (int64_t)tm * BM + r;
    const uint32_t bias = 1024u * (uint32_t)(i % 4);
    kb[i] = c * 16 < krem;
    ob[i] = ((r < BM && row < M) ? (uint32_t)(row * K + c * 16) : kOOB) - bias;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t la0 = lds0 + (uint32_t)(wid * NA) * 1024u;
  const uint32_t lb0 = lds0 + (uint32_t)(IA + wid * NB) * 1024u;
  const bool small_k = K < BK;

  // Issue M0 group g (0 <= g < NG) of the copies of K step ks into `slot`.
  auto issue_group = [&](int g, int slot, int ks) {
    const int soff = ks * BK;
    const uint32_t so = (uint32_t)(slot * STAGE);
    const bool tail = ktail && ks + 1 == p.nks;
    const bool isA = g < GA;
    const int i0 = (isA ? g : g - GA) * 4;
    const uint32_t base = (isA ? la0 : lb0) + so + (uint32_t)i0 * 1024u;
    uint32_t vo[4];
    auto run = [&](auto cnt_c) {
      constexpr int C = decltype(cnt_c)::value;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        const int i = i0 + e;
        const uint32_t o = isA ? oa[i] : ob[i];
        const bool k_ok = isA ? ka[i] : kb[i];
        vo[e] = (!tail || k_ok) ? o : kOOB - 1024u * (uint32_t)e;
      }
      if (small_k) {
        // K < 128: the first rows' biased offsets would wrap below zero, so
        // each copy gets its own M0 and an unbiased offset.
#pragma unroll
        for (int e = 0; e < C; ++e) {
          const uint32_t u = vo[e] + 1024u * (uint32_t)e;
          if (isA) dma_group<1, NTW>(base + 1024u * (uint32_t)e, &u, rsw, soff);
          else dma_group<1, false>(base + 1024u * (uint32_t)e, &u, rsx, soff);
        }
      } else {
        if (isA) dma_group<C, NTW>(base, vo, rsw, soff);
        else dma_group<C, false>(base, vo, rsx, soff);
      }
    };
    const int cnt = isA ? (NA - i0 < 4 ? NA - i0 : 4) : (NB - i0 < 4 ? NB - i0 : 4);
    if (cnt == 4) run(std::integral_constant<int, 4>{});
    else if (cnt == 3) run(std::integral_constant<int, 3>{});
    else if (cnt == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  };
  auto issue_all = [&](int slot, int ks) {
#pragma unroll
    for (int g = 0; g < NG; ++g) issue_group(g, slot, ks);
  };

  // ---- MFMA fragment reads
  const int lr = lane % T;
  const int lg = (lane / T) * (LB / 16);
  const int sl = swz<BK>(lr);
  const int rbaseA = (wn * WTN + lr) * BK;
  const int rbaseB = IA * 1024 + (wm * WTM + lr) * BK;
  int xo0[NKK], xo1[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int c0 = kk * (KI / 16) + lg;
    xo0[kk] = (c0 ^ sl) << 4;
    xo1[kk] = ((c0 + 1) ^ sl) << 4;
  }
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
  // MFMAs of one K step; the copy groups of a later step (if any) are
  // spread over its NKK sub-steps.
  auto compute = [&](int slot, bool do_issue, int islot, int iks) {
    const uint8_t* A = smem + slot * STAGE + rbaseA;
    const uint8_t* B = smem + slot * STAGE + rbaseB;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      op_t a[FN], bb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) a[i] = lds_op(A + i * T * BK, kk);
#pragma unroll
      for (int j = 0; j < FM; ++j) bb[j] = lds_op(B + j * T * BK, kk);
      if (do_issue) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
          if (g * NKK / NG == kk) issue_group(g, islot, iks);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::run(a[i], bb[j], acc[i][j]);
    }
  };

  // ---- main loop. K step ks0 + it lives in slot it % S. At the top of step
  // it the copies of steps up to it + S - 2 have been issued; this wave
  // waits for its copies of step it, the barrier makes every wave's copies
  // visible and guarantees slot (it - 1) % S is no longer read, and the
  // copies of step it + S - 1 go into that slot while the MFMAs of step it
  // run.
  // Scales are loaded before the K loop unless the accumulators already
  // take 128 or more registers per lane (the 256 x 256 tile would spill).
  constexpr bool kEarlyScales = FN * FM * MF::NACC < 128;
  EpiScales<FN, FM, MF::NACC / 4> sc;
  if constexpr (kEarlyScales) load_scales<QT, T, BN, BM, WN, WM>(p, tn, tm, wn, wm, lane, sc);
  uint32_t g0 = 0;  // fused launches: barrier generation at launch start
  if constexpr (FUSE) g0 = fuse_generation(p.f.bar);

  const int nk = ks1 - ks0;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue_all(s, ks0 + s);
  int cs = 0, is = S - 1;
  for (int it = 0; it < nk; ++it) {
    wait_stages<NI, S - 2>(nk - 1 - it);
    __syncthreads();
    compute(cs, it + S - 1 < nk, is, ks0 + it + S - 1);
    cs = cs + 1 == S ? 0 : cs + 1;
    is = is + 1 == S ? 0 : is + 1;
  }

  if constexpr (!kEarlyScales) load_scales<QT, T, BN, BM, WN, WM>(p, tn, tm, wn, wm, lane, sc);

  constexpr int LDT = BN + 4;  // staged row stride in bf16 (8 bytes of padding)
  constexpr int CHF = (S * STAGE) / (LDT * 2);      // tokens that fit the ring
  constexpr int CH0 = CHF >= BM ? BM : CHF / WTM * WTM;  // chunk: whole wave tiles
  if constexpr (FUSE) {
    if (p.splitk > 1) {
      store_partials_dev<QT, T, BN, BM, WN, WM>(p, acc, tn, tm, z, wn, wm, lane);
      fused_splitk_tail<QT, NW>(p, g0, wid, lane);
    } else {
      fused_direct_tail<QT, T, BN, BM, WN, WM, LDT, CH0>(p, acc, sc, smem, g0, tn, tm, wn, wm,
                                                          lane, tid);
    }
    return;
  }

  // bf16 outputs go through LDS (the ring is free once every wave is past
  // its last K step), so each lane stores 16 contiguous bytes of a token's
  // row: the MFMA layout would make every store instruction write 8 bytes
  // into each of 32 rows. Split partial sums, raw accumulators and row
  // strides that are not a multiple of 8 take the direct path.
  if constexpr (CH0 >= WTM) {
    if (p.splitk == 1 && !p.out_raw && (p.ldy & 7) == 0) {
      store_tile_staged<QT, T, BN, BM, WN, WM, LDT, CH0>(p, acc, sc, smem, tn, tm, wn, wm, lane,
                                                          tid);
      return;
    }
  }
  store_tile<QT, T, BN, BM, WN, WM>(p, acc, sc, tn, tm, z, wn, wm, lane);
}

// Split-K second pass: Y[m, n] = epilogue(sum_{z = 0..S-1} part[z][m][n]),
// summed in split order. One thread per four consecutive n of one m. With the
// split count SC known at compile time (2..8, every count the planner makes)
// the partials are loaded together before they are added; SC = 0 takes S at
// run time and loads one split after another.
template <int QT, int SC>
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
  auto add = [&](const uint32_t (&w)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (QT == kQInt8) si[e] += (int32_t)w[e];
      else sf[e] += __uint_as_float(w[e]);
    }
  };
  auto load = [&](int zz, uint32_t (&w)[4]) {
    const uint32_t* src = part + (int64_t)zz * M * N + m * N + n0;
    if (v4) {
      const uint4 u = *reinterpret_cast<const uint4*>(src);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      w[0] = w[1] = w[2] = w[3] = 0u;
      for (int e = 0; e < cnt; ++e) w[e] = src[e];
    }
  };
  if constexpr (SC > 0) {
    uint32_t w[SC][4];
    if (v4) {
#pragma unroll
      for (int q = 0; q < SC; ++q) {
        const uint4 u = *reinterpret_cast<const uint4*>(part + (int64_t)q * M * N + m * N + n0);
        w[q][0] = u.x; w[q][1] = u.y; w[q][2] = u.z; w[q][3] = u.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < SC; ++q) load(q, w[q]);
    }
#pragma unroll
    for (int q = 0; q < SC; ++q) add(w[q]);
  } else {
    for (int zz = 0; zz < S; ++zz) {
      uint32_t w[4];
      load(zz, w);
      add(w);
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

// Split-K sum with the bf16 epilogue, eight consecutive outputs of one token
// per thread (N % 8 == 0, ldy % 8 == 0, Y 16-byte aligned): the same sums in
// split order and the same epilogue as splitk_reduce_kernel, one 16-byte store.
template <int QT, int SC>
__global__ __launch_bounds__(256) void splitk_reduce8_kernel(
    const uint32_t* __restrict__ part, int64_t M, int64_t N, const float* __restrict__ sx,
    const float* __restrict__ sw, uint16_t* __restrict__ Y, int64_t ldy) {
  const int64_t ng = N >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * ng) return;
  const int64_t m = idx / ng, n0 = (idx % ng) * 8;
  uint32_t w[SC][8];
#pragma unroll
  for (int z = 0; z < SC; ++z) {
    const uint4* src = reinterpret_cast<const uint4*>(part + (int64_t)z * M * N + m * N + n0);
    const uint4 a = src[0], b = src[1];
    w[z][0] = a.x; w[z][1] = a.y; w[z][2] = a.z; w[z][3] = a.w;
    w[z][4] = b.x; w[z][5] = b.y; w[z][6] = b.z; w[z][7] = b.w;
  }
  const float sxm = sx[m];
  uint32_t bb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc;
    if constexpr (QT == kQInt8) {
      int32_t si = 0;
#pragma unroll
      for (int z = 0; z < SC; ++z) si += (int32_t)w[z][e];
      acc = (float)si;
    } else {
      float sf = 0.0f;
#pragma unroll
      for (int z = 0; z < SC; ++z) sf += __uint_as_float(w[z][e]);
      acc = sf;
    }
    bb[e] = epi_bf16(acc, sxm, sw[n0 + e]);
  }
  *reinterpret_cast<uint4*>(Y + m * ldy + n0) =
      make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                 bb[6] | (bb[7] << 16));
}

// Split-K sum that also quantizes the next linear's input: one block per
// token row m. Each thread owns groups of 8 consecutive outputs (16 bytes of
// bf16), n = 8 (t + 256 i): it adds the S partial sums of the group in split
// order (as splitk_reduce_kernel does), applies the bf16 epilogue, stores the
// group to Y and keeps it in registers; then the row's absmax over the
// quantized columns [q0, q0 + qn) and their codes follow the per-token
// quantizer's arithmetic on those same bf16 values (absmax8_bf16,
// t = absmax / Q, codes8_bf16, scale t * act_mult), so Y, the codes and the
// scale equal the reduction kernel followed by the quantizer bit for bit.
// Requires N % 8 == 0, ldy % 8 == 0, q0 and qn multiples of 8, and
// N <= 2048 G.
template <int QT, int SC, int G>
__global__ __launch_bounds__(256) void splitk_reduce_quant_kernel(
    const uint32_t* __restrict__ part, int64_t M, int64_t N, const float* __restrict__ sx,
    const float* __restrict__ sw, uint16_t* __restrict__ Y, int64_t ldy, int64_t q0, int64_t qn,
    float act_mult, uint8_t* __restrict__ Xq, float* __restrict__ scale_x) {
  static_assert(SC >= 2 && SC <= 8, "splits");
  __shared__ float red[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t m = blockIdx.x;
  const int64_t ng = N >> 3;
  const float sxm = sx[m];
  uint4 v[G];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int64_t g = t + 256 * (int64_t)i;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (g >= ng) continue;
    const int64_t n0 = 8 * g;
    uint32_t w[SC][8];
#pragma unroll
    for (int z = 0; z < SC; ++z) {
      const uint4* src = reinterpret_cast<const uint4*>(part + (int64_t)z * M * N + m * N + n0);
      const uint4 a = src[0], b = src[1];
      w[z][0] = a.x; w[z][1] = a.y; w[z][2] = a.z; w[z][3] = a.w;
      w[z][4] = b.x; w[z][5] = b.y; w[z][6] = b.z; w[z][7] = b.w;
    }
    uint32_t bb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc;
      if constexpr (QT == kQInt8) {
        int32_t si = 0;
#pragma unroll
        for (int z = 0; z < SC; ++z) si += (int32_t)w[z][e];
        acc = (float)si;
      } else {
        float sf = 0.0f;
#pragma unroll
        for (int z = 0; z < SC; ++z) sf += __uint_as_float(w[z][e]);
        acc = sf;
      }
      bb[e] = epi_bf16(acc, sxm, sw[n0 + e]);
    }
    v[i] = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                      bb[6] | (bb[7] << 16));
    *reinterpret_cast<uint4*>(Y + m * ldy + n0) = v[i];
    if (n0 >= q0 && n0 < q0 + qn) amax = fmaxf(amax, absmax8_bf16(v[i]));
  }
  if (qn == 0) return;
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float tq = amax / qmax<QT>();
  if (t == 0) scale_x[m] = tq * act_mult;
  uint2* qrow = reinterpret_cast<uint2*>(Xq + m * qn);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int64_t n0 = 8 * (t + 256 * (int64_t)i);
    if (n0 >= N || n0 < q0 || n0 >= q0 + qn) continue;
    qrow[(n0 - q0) >> 3] = tq == 0.0f ? make_uint2(0u, 0u) : codes8_bf16<QT>(v[i], tq);
  }
}

// ---------------------------------------------------------------------------
// Tile table. Order matters: the planner and the tuning hook refer to tiles
// by index. (S, T, BN, BM, WN, WM, BK, FU): S is the LDS ring depth, T the
// MFMA edge, BN x BM the macro tile over N and M, WN x WM the waves along N
// and M, BK the bytes of K per step, FU 1 when the tile also has a fused
// chain-epilogue instantiation (the tiles the planner picks up to 1024
// tokens), NT 1 when the weight copies carry the non-temporal hint: weight
// bytes are streamed once (measured 3-6% faster at 1, 32 and 512 tokens);
// the 192 x 128 tile reads each weight tile twice (two token tiles, one
// after the other on the same XCD) and the hint made it 5% slower, so its
// second read would not hit in L2. The kernel also takes 64-byte K steps (twice the ring slots in
// the same LDS); measured on the 32B-shaped GEMMs at 512 and 4096 tokens,
// 256 x 256 and 256 x 128 tiles with 64-byte steps and rings of 4-6 were
// 2-15% slower than their 128-byte versions, so no tile uses them.
// ---------------------------------------------------------------------------
#define QR_TILES(X)                                                                \
  X(4, 16, 128, 32, 8, 1, 128, 1, 1)  /*  0: M <= 32, weight streaming        */ \
  X(4, 32, 128, 64, 4, 2, 128, 1, 1)  /*  1: M <= 64; narrow 256-token layers */ \
  X(4, 32, 128, 128, 2, 4, 128, 1, 1) /*  2: M <= 128; long-K 256-token ones  */ \
  X(3, 32, 256, 128, 4, 2, 128, 1, 1) /*  3: long-K / narrow large-M layers   */ \
  X(2, 32, 256, 256, 2, 4, 128, 0, 1) /*  4: wide large-M layers              */ \
  X(3, 32, 128, 256, 2, 4, 128, 1, 1) /*  5: 256-token very wide layers       */ \
  X(4, 32, 128, 32, 4, 1, 128, 1, 1)  /*  6: M <= 32 narrow layers, 4 waves   */ \
  X(6, 16, 64, 16, 4, 1, 128, 1, 1)   /*  7: M <= 16 narrow layers            */ \
  X(4, 32, 192, 128, 2, 4, 128, 1, 0) /*  8: wide 256-token layers, 8 waves   */ \
  X(4, 16, 80, 64, 5, 1, 128, 1, 1)   /*  9: 256-token INT8 QKV, 5 waves      */ \
  X(2, 32, 192, 256, 2, 4, 128, 0, 1) /* 10: 256-token stacked gate + up      */

#define QR_STR(x) #x
#define QR_DESC(S, T, BN, BM, WN, WM, BK, FU, NT)                                          \
  {BK == 64 ? "dma" QR_STR(S) "_t" #T "_n" #BN "_m" #BM "_w" #WN "x" #WM "_k64"         \
            : "dma" QR_STR(S) "_t" #T "_n" #BN "_m" #BM "_w" #WN "x" #WM,               \
   T, BN, BM, BK, 64 * WN * WM, S, FU},
const TileDesc kTiles[] = {QR_TILES(QR_DESC)};
#undef QR_DESC
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int QT, int S, int T, int BN, int BM, int WN, int WM, int BK, int NT>
hipError_t launch_one(const KParams& kp, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_dma_kernel<QT, T, BN, BM, WN, WM, S, BK, NT == 1, false>), dim3(grid),
                     dim3(64 * WN * WM), 0, st, kp);
  return hipGetLastError();
}

// Fused-epilogue kernel of a tile: its function (for the residency check) or
// its launch.
template <int QT, int S, int T, int BN, int BM, int WN, int WM, int BK, int FU, int NT>
const void* fused_fn() {
  if constexpr (FU == 1)
    return reinterpret_cast<const void*>(
        &gemm_dma_kernel<QT, T, BN, BM, WN, WM, S, BK, NT == 1, true>);
  else
    return nullptr;
}
template <int QT, int S, int T, int BN, int BM, int WN, int WM, int BK, int FU, int NT>
hipError_t launch_fused_one(const KParams& kp, unsigned grid, hipStream_t st) {
  if constexpr (FU == 1) {
    hipLaunchKernelGGL((gemm_dma_kernel<QT, T, BN, BM, WN, WM, S, BK, NT == 1, true>), dim3(grid),
                       dim3(64 * WN * WM), 0, st, kp);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

}  // namespace

int num_tiles() { return kNumTiles; }
const TileDesc& tile_desc(int tile) { return kTiles[tile]; }

hipError_t launch_gemm(const GemmPlan& plan, int qt, const GemmArgs& a, hipStream_t st, bool sum_splits) {
  KParams kp;
  kp.Xq = a.Xq; kp.sx = a.sx; kp.Wq = a.Wq; kp.sw = a.sw;
  kp.M = a.M; kp.N = a.N; kp.K = a.K;
  kp.splitk = plan.splitk;
  kp.tiles_n = (int)plan.tiles_n; kp.tiles_m = (int)plan.tiles_m; kp.nks = (int)plan.nks;
  kp.rn = plan.rows;
  if (plan.splitk > 1) {
    kp.Y = a.part; kp.ldy = a.N; kp.out_raw = 1; kp.vec = (a.N % 4) == 0;
  } else {
    kp.Y = a.Y; kp.ldy = a.ldy; kp.out_raw = a.out_raw; kp.vec = (a.ldy % 4) == 0;
  }
  const unsigned grid = (unsigned)(plan.tiles_n * plan.tiles_m * plan.splitk);
  hipError_t e = hipErrorInvalidValue;
  int idx = 0;
#define QR_CASE(S, T, BN, BM, WN, WM, BK, FU, NT)                                  \
  if (plan.tile == idx) {                                                           \
    e = qt == kQInt8 ? launch_one<kQInt8, S, T, BN, BM, WN, WM, BK, NT>(kp, grid, st) \
                     : launch_one<kQFp8, S, T, BN, BM, WN, WM, BK, NT>(kp, grid, st); \
  }                                                                                 \
  ++idx;
  QR_TILES(QR_CASE)
#undef QR_CASE
  if (e != hipSuccess || plan.splitk <= 1 || !sum_splits) return e;
  const int64_t work = a.M * ((a.N + 3) / 4);
  const unsigned rgrid = (unsigned)((work + 255) / 256);
  const int vec = (a.ldy % 4) == 0;
  // bf16 outputs with N and ldy multiples of 8 and Y 16-byte aligned: eight
  // outputs per thread and one 16-byte store (measured 1-4 us faster on the
  // 256- and 512-token down projections, the same bits); otherwise four.
  const bool by8 = !a.out_raw && a.N % 8 == 0 && a.ldy % 8 == 0 &&
                   (reinterpret_cast<uintptr_t>(a.Y) & 15) == 0;
  const unsigned rgrid8 = (unsigned)((a.M * (a.N / 8) + 255) / 256);
  auto reduce = [&](auto qt_c, auto sc_c) {
    constexpr int Q = decltype(qt_c)::value, SC = decltype(sc_c)::value;
    if constexpr (SC >= 2) {
      if (by8) {
        hipLaunchKernelGGL((splitk_reduce8_kernel<Q, SC>), dim3(rgrid8), dim3(256), 0, st,
                           static_cast<const uint32_t*>(a.part), a.M, a.N, a.sx, a.sw,
                           static_cast<uint16_t*>(a.Y), a.ldy);
        return;
      }
    }
    hipLaunchKernelGGL((splitk_reduce_kernel<Q, SC>), dim3(rgrid), dim3(256), 0, st,
                       static_cast<const uint32_t*>(a.part), plan.splitk, a.M, a.N, a.sx, a.sw,
                       a.Y, a.ldy, a.out_raw, vec);
  };
  auto by_splits = [&](auto qt_c) {
    switch (plan.splitk) {
      case 2: reduce(qt_c, std::integral_constant<int, 2>{}); break;
      case 3: reduce(qt_c, std::integral_constant<int, 3>{}); break;
      case 4: reduce(qt_c, std::integral_constant<int, 4>{}); break;
      case 5: reduce(qt_c, std::integral_constant<int, 5>{}); break;
      case 6: reduce(qt_c, std::integral_constant<int, 6>{}); break;
      case 7: reduce(qt_c, std::integral_constant<int, 7>{}); break;
      case 8: reduce(qt_c, std::integral_constant<int, 8>{}); break;
      default: reduce(qt_c, std::integral_constant<int, 0>{}); break;
    }
  };
  if (qt == kQInt8) by_splits(std::integral_constant<int, kQInt8>{});
  else by_splits(std::integral_constant<int, kQFp8>{});
  return hipGetLastError();
}

bool splitk_reduce_quant_ok(int64_t N, int splitk) {
  return splitk >= 2 && splitk <= 8 && N % 8 == 0 && N <= 8 * 2048;
}

hipError_t launch_splitk_reduce_quant(int splitk, int qt, const void* part, int64_t M, int64_t N,
                                      const float* sx, const float* sw, void* Y, int64_t ldy,
                                      int64_t q0, int64_t qn, float act_mult, void* Xq,
                                      float* scale_x, hipStream_t st) {
  if (!splitk_reduce_quant_ok(N, splitk) || M <= 0) return hipErrorInvalidValue;
  const int G = N <= 2 * 2048 ? 2 : N <= 4 * 2048 ? 4 : 8;
  auto go = [&](auto qt_c, auto sc_c, auto g_c) {
    constexpr int Q = decltype(qt_c)::value, SC = decltype(sc_c)::value, GG = decltype(g_c)::value;
    hipLaunchKernelGGL((splitk_reduce_quant_kernel<Q, SC, GG>), dim3((unsigned)M), dim3(256), 0, st,
                       static_cast<const uint32_t*>(part), M, N, sx, sw, static_cast<uint16_t*>(Y),
                       ldy, q0, qn, act_mult, static_cast<uint8_t*>(Xq), scale_x);
  };
  auto by_g = [&](auto qt_c, auto sc_c) {
    if (G == 2) go(qt_c, sc_c, std::integral_constant<int, 2>{});
    else if (G == 4) go(qt_c, sc_c, std::integral_constant<int, 4>{});
    else go(qt_c, sc_c, std::integral_constant<int, 8>{});
  };
  auto by_s = [&](auto qt_c) {
    switch (splitk) {
      case 2: by_g(qt_c, std::integral_constant<int, 2>{}); break;
      case 3: by_g(qt_c, std::integral_constant<int, 3>{}); break;
      case 4: by_g(qt_c, std::integral_constant<int, 4>{}); break;
      case 5: by_g(qt_c, std::integral_constant<int, 5>{}); break;
      case 6: by_g(qt_c, std::integral_constant<int, 6>{}); break;
      case 7: by_g(qt_c, std::integral_constant<int, 7>{}); break;
      default: by_g(qt_c, std::integral_constant<int, 8>{}); break;
    }
  };
  if (qt == kQInt8) by_s(std::integral_constant<int, kQInt8>{});
  else by_s(std::integral_constant<int, kQFp8>{});
  return hipGetLastError();
}

namespace {

// Items of 256 outputs of one token per wave of a split plan's fused sum.
int64_t fused_items_per_wave(const GemmPlan& plan, int64_t M, int64_t N) {
  const int64_t waves = plan.tiles_n * plan.tiles_m * plan.splitk * (tile_desc(plan.tile).NT / 64);
  const int64_t items = M * ((N + 255) / 256);
  return (items + waves - 1) / waves;
}

// Blocks of the fused kernel of (tile, qt) one CU holds at once (0 if it
// has none); queried once per device and cached.
int fused_blocks_per_cu(int tile, int qt, int dev) {
  constexpr int kDevs = 16;
  static int cache[kDevs][2][32];  // 0: not queried yet; else 1 + blocks
  if (dev < 0 || dev >= kDevs || tile < 0 || tile >= 32) return 0;
  int& c = cache[dev][qt == kQInt8 ? 0 : 1][tile];
  if (c == 0) {
    const void* fn = nullptr;
    int idx = 0;
#define QR_FN(S, T, BN, BM, WN, WM, BK, FU, NT)                                        \
  if (tile == idx)                                                                    \
    fn = qt == kQInt8 ? fused_fn<kQInt8, S, T, BN, BM, WN, WM, BK, FU, NT>()          \
                      : fused_fn<kQFp8, S, T, BN, BM, WN, WM, BK, FU, NT>();          \
  ++idx;
    QR_TILES(QR_FN)
#undef QR_FN
    int nb = 0;
    if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, tile_desc(tile).NT, 0) !=
                  hipSuccess)
      nb = 0;
    c = 1 + nb;
  }
  return c - 1;
}

}  // namespace

bool fused_ok(const GemmPlan& plan, int qt, int64_t M, int64_t N) {
  if (plan.tile < 0 || plan.tile >= kNumTiles || !kTiles[plan.tile].FU) return false;
  if (M > kFuseMaxM || M <= 0 || N <= 0) return false;
  if (plan.splitk > 1 && fused_items_per_wave(plan, M, N) > kFuseItems) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  const int64_t grid = plan.tiles_n * plan.tiles_m * plan.splitk;
  return grid <= (int64_t)cus * fused_blocks_per_cu(plan.tile, qt, dev);
}

hipError_t launch_gemm_fused(const GemmPlan& plan, int qt, const GemmArgs& a, const FuseArgs& fa,
                             hipStream_t st) {
  KParams kp;
  kp.Xq = a.Xq; kp.sx = a.sx; kp.Wq = a.Wq; kp.sw = a.sw;
  kp.M = a.M; kp.N = a.N; kp.K = a.K;
  kp.splitk = plan.splitk;
  kp.tiles_n = (int)plan.tiles_n; kp.tiles_m = (int)plan.tiles_m; kp.nks = (int)plan.nks;
  kp.rn = plan.rows;
  uint32_t* hdr = static_cast<uint32_t*>(fa.header);
  kp.f.bar = hdr;
  kp.f.pmax = hdr + 64;  // 256 bytes in
  kp.f.part = static_cast<uint32_t*>(fa.part);
  kp.f.xq2 = fa.xq2; kp.f.sx2 = fa.sx2;
  kp.f.qc0 = fa.qc0; kp.f.qcn = fa.qcn; kp.f.am2 = fa.am2;
  kp.f.ipw = plan.splitk > 1 ? (int)fused_items_per_wave(plan, a.M, a.N) : 0;
  kp.f.y = static_cast<uint16_t*>(a.Y); kp.f.ldy = a.ldy;
  if (plan.splitk > 1) {
    kp.Y = fa.part; kp.ldy = a.N; kp.out_raw = 1; kp.vec = (a.N % 4) == 0;
  } else {
    kp.Y = a.Y; kp.ldy = a.ldy; kp.out_raw = 0; kp.vec = (a.ldy % 4) == 0;
  }
  const unsigned grid = (unsigned)(plan.tiles_n * plan.tiles_m * plan.splitk);
  hipError_t e = hipErrorInvalidValue;
  int idx = 0;
#define QR_FCASE(S, T, BN, BM, WN, WM, BK, FU, NT)                                            \
  if (plan.tile == idx) {                                                                      \
    e = qt == kQInt8 ? launch_fused_one<kQInt8, S, T, BN, BM, WN, WM, BK, FU, NT>(kp, grid, st) \
                     : launch_fused_one<kQFp8, S, T, BN, BM, WN, WM, BK, FU, NT>(kp, grid, st); \
  }                                                                                            \
  ++idx;
  QR_TILES(QR_FCASE)
#undef QR_FCASE
  return e;
}

}  // namespace qr
