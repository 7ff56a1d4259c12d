// Block-wise FP8 for gfx950: E4M3FN elements with one power-of-two (E8M0)
// scale per 32 consecutive elements of a row, the scaling the CDNA4 matrix
// cores apply natively (v_mfma_scale_f32_16x16x128_f8f6f4 takes one scale
// byte per row and 32-element block of K). The block-wise variant is
// the one the QuRL pages cite ([fugumt] "Related papers": FP8-RL); its block
// size and scale format are not on the pages, and these are the hardware's.
//
//   mx_quant_kernel  one thread per 32-element block: absmax, exponent X (the
//                    smallest with absmax <= 448 * 2^X), the E8M0 byte X + 127,
//                    and the codes of fl32(v * 2^-X). Scale bytes are stored in
//                    panels of 128 elements of K: [ceil(K / 128)][R][4], so the
//                    four bytes a row needs for one 128-byte K step sit together
//                    and a tile's bytes for that step are one contiguous run.
//   mx_dma_kernel    weights on the MFMA A operand, tokens on B; code tiles
//                    and their scale bytes move global -> LDS with LDS-DMA
//                    copies into an S-slot ring (one barrier per 128-byte K
//                    step), so the tokens are fetched once per block and
//                    shared by its 8 waves; output bf16(acc) or the fp32
//                    accumulators.
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWordBuf = 0x00020000;  // raw buffer resource word 3 (gfx9)

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
  scales[((b >> 2) * R + row) * 4 + (b & 3)] = (uint8_t)(X + 127);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = mx_codes4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], -X);
  uint4* out = reinterpret_cast<uint4*>(codes + row * K + b * 32);
  out[0] = make_uint4(q[0], q[1], q[2], q[3]);
  out[1] = make_uint4(q[4], q[5], q[6], q[7]);
}

// ---------------------------------------------------------------------------
// LDS-DMA block-scaled GEMM. A stage holds, for one 128-byte K step, the
// weight rows of the tile (BN x 128 bytes), the token rows (BM x 128 bytes,
// padded to whole 1 KB blocks per wave) and the four E8M0 bytes of every
// row's 32-element blocks in that step (4 bytes per row; 1 KB for up to 256
// weight rows, then 1 KB for up to 256 token rows). Code rows are copied 8
// rows (1 KB) per wave instruction with buffer_load_dwordx4 ... lds (64 lanes
// x 16 bytes at M0 + offset + 16 lane; up to four copies share one M0 write
// through the instruction offset). The scale bytes of a step are stored
// contiguously per operand (panels [K / 128][rows][4]), so wave 0 copies the
// weight tile's and wave 1 the token tile's with one such instruction each;
// a wave waits for its own copies with a fixed vmcnt (one more for waves 0
// and 1), and one barrier per K step publishes them. 16-byte LDS chunks are XOR-swizzled by row (chunk c of row r sits at
// c ^ ((r >> 1) & 7)), applied on the global side of the copy.
//
// In the 16x16x128 scaled MFMA, lane l (row l % 16, group g = l / 16) holds
// K bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of the step and
// the scale byte of 32-element block g of its row (the hardware's layout,
// measured), so a lane reads LDS chunks g and g + 4 of its row and scale byte
// g. The 32x32x64 form (two per 128-byte step, sub-step h) follows the same
// pattern with two lane groups: lane l (row l % 32, g = l / 32) holds K bytes
// [64 h + 16 g, + 16) and [64 h + 32 + 16 g, + 16) and the scale of block
// 2 h + g (checked by the parity tests against exact block sums). A tile may own fewer weight rows than its height (rn, a multiple of 8)
// so the grid can be balanced over the CUs; rows past rn or N read as zero
// and are not stored.
// ---------------------------------------------------------------------------
struct MxDmaParams {
  const uint8_t* Xq;
  const uint8_t* sx;
  const uint8_t* Wq;
  const uint8_t* sw;
  int64_t M, N, K;
  void* Y;
  int64_t ldy;
  int out_raw;
  int tiles_m, nks, rn;
};

template <int CNT>
__device__ __forceinline__ void mx_dma16(uint32_t lds, const uint32_t* vo,
                                         __amdgpu_buffer_rsrc_t r, int soff) {
  static_assert(CNT >= 1 && CNT <= 4, "one M0 covers at most 4 KB of offsets");
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (CNT == 1)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(vo[0]), "s"(r), "s"(soff) : "memory", "m0");
  else if constexpr (CNT == 2)
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds"
                 :: "s"(lds), "v"(vo[0]), "v"(vo[1]), "s"(r), "s"(soff) : "memory", "m0");
  else if constexpr (CNT == 3)
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %1, %4, %5 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %4, %5 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %4, %5 offen offset:2048 lds"
                 :: "s"(lds), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "s"(r), "s"(soff)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
                 :: "s"(lds), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(r), "s"(soff)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

template <int N>
__device__ __forceinline__ void mx_wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most min(ahead, A) stages of NI copies are in flight.
template <int NI, int A>
__device__ __forceinline__ void mx_wait_stages(int ahead) {
  if constexpr (A > 0) {
    if (ahead >= A) {
      mx_wait_vm<A * NI>();
      return;
    }
    mx_wait_stages<NI, A - 1>(ahead);
  } else {
    mx_wait_vm<0>();
  }
}

template <int T>
struct MxMfma;
template <>
struct MxMfma<16> {
  using acc_t = v4f;
  static constexpr int KI = 128;
  static __device__ __forceinline__ acc_t run(v8i a, v8i b, acc_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  }
};
template <>
struct MxMfma<32> {
  using acc_t = v16f;
  static constexpr int KI = 64;
  static __device__ __forceinline__ acc_t run(v8i a, v8i b, acc_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  }
};

// bf16 outputs staged through LDS: every lane converts its groups of four
// outputs (four consecutive channels of one token) and writes them, 8 bytes,
// to a [CH][LDT] bf16 tile; then the block stores the owned channels of each
// token as 16-byte pieces (the N tail one by one). Tiles whose tokens do not
// all fit the LDS go in chunks of CH tokens, a multiple of the wave tile's.
// Requires ldy % 8 == 0; the tile's first channel tn * rn is a multiple of 8
// and Y is 16-byte aligned (both checked by the host), so every full piece is
// an aligned 16-byte store.
template <int T, int BN, int BM, int WN, int WM, int LDT, int CH, typename acc_t, int FN, int FM>
__device__ __forceinline__ void mx_store_staged(const MxDmaParams& p, const acc_t (&acc)[FN][FM],
                                                uint8_t* smem, int tn, int tm, int wn, int wm,
                                                int lane, int tid) {
  constexpr int NT = 64 * WN * WM;
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int NR = T == 16 ? 4 : 16;
  static_assert((LDT * 2) % 8 == 0, "8-byte aligned staged rows");
  static_assert(CH % WTM == 0 && CH >= WTM && CH <= BM, "chunks of whole wave tiles");
  uint16_t* so = reinterpret_cast<uint16_t*>(smem);
  const int64_t N = p.N, M = p.M;
  const int64_t n0 = (int64_t)tn * p.rn;
  const int own = (int)((N - n0) < p.rn ? (N - n0) : p.rn);  // owned output channels
  const int mv = (int)((M - (int64_t)tm * BM) < BM ? (M - (int64_t)tm * BM) : BM);
  const int cpt = (own + 7) / 8;  // 16-byte pieces per token row
  const int lr = lane % T, lg = lane / T;
  uint16_t* Y = static_cast<uint16_t*>(p.Y) + ((int64_t)tm * BM) * p.ldy + n0;
#pragma unroll
  for (int c0 = 0; c0 < BM; c0 += CH) {
    __syncthreads();  // the operand ring (first chunk) or the last chunk is no longer read
    if (wm * WTM >= c0 && wm * WTM < c0 + CH) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int ml = wm * WTM + T * j + lr - c0;  // token within the chunk
#pragma unroll
          for (int q = 0; q < NR / 4; ++q) {
            const int nl = wn * WTN + T * i + 8 * q + 4 * lg;  // local channel of register 4 q
            uint32_t bb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) bb[r] = f32_to_bf16_rne(acc[i][j][4 * q + r]);
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
        const uint2 lo = *reinterpret_cast<const uint2*>(src);
        const uint2 hi = *reinterpret_cast<const uint2*>(src + 4);
        *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        for (int e = 0; nl + e < own; ++e) dst[e] = src[e];
      }
    }
  }
}

template <int T, int BN, int BM, int WN, int WM, int S>
__global__ __launch_bounds__(64 * WN * WM, 1) void mx_dma_kernel(const MxDmaParams p) {
  using MF = MxMfma<T>;
  using acc_t = typename MF::acc_t;
  constexpr int KI = MF::KI, NKK = 128 / KI;
  constexpr int NW = WN * WM;
  constexpr int WTN = BN / WN, WTM = BM / WM;
  constexpr int FN = WTN / T, FM = WTM / T;
  constexpr int IA = BN / 8;
  constexpr int IB0 = BM / 8;
  constexpr int IB = IB0 + (NW - IB0 % NW) % NW;
  constexpr int NA = IA / NW, NB = IB / NW;
  constexpr int NI = NA + NB;  // code copies per wave per K step
  constexpr int GA = (NA + 3) / 4, GB = (NB + 3) / 4;
  constexpr int CODES = (IA + IB) * 1024;
  constexpr int STAGE = CODES + 2048;  // + weight and token scale bytes
  static_assert(BN % 16 == 0 && BM % 16 == 0 && IA % NW == 0, "row blocks per wave");
  static_assert(WTN % T == 0 && WTM % T == 0, "wave tile");
  static_assert(BN <= 256 && BM <= 256 && NW >= 2, "one scale copy per operand");
  static_assert(S >= 2 && (S - 2) * (NI + 1) <= 63, "ring depth");
  static_assert(S * STAGE <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int G = gridDim.x;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);  // neighbouring tiles on one XCD
  const int tm = b % p.tiles_m, tn = b / p.tiles_m;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wid % WN, wm = wid / WN;
  const int64_t N = p.N, M = p.M, K = p.K, nb = K >> 5;
  constexpr uint32_t kBig = 0x80000000u;

  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Wq, (short)0, (int)(uint32_t)(N * K), kWordBuf);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Xq, (short)0, (int)(uint32_t)(M * K), kWordBuf);
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.sw, (short)0, (int)(uint32_t)(N * nb), kWordBuf);
  const __amdgpu_buffer_rsrc_t rsx =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.sx, (short)0, (int)(uint32_t)(M * nb), kWordBuf);

  // Code copies: wave wid moves weight row blocks wid*NA + i and token row
  // blocks wid*NB + i; lane l covers row 8 rb + l / 8, physical chunk l % 8.
  // Offsets are biased by -1 KB * (i % 4), the copy's instruction offset.
  const int lrow = lane >> 3, pch = lane & 7;
  uint32_t oa[NA], ob[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = (wid * NA + i) * 8 + lrow;
    const int c = pch ^ ((r >> 1) & 7);
    const int64_t row = (int64_t)tn * p.rn + r;
    oa[i] = ((r < p.rn && row < N) ? (uint32_t)(row * K + c * 16) : kBig) - 1024u * (uint32_t)(i % 4);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = (wid * NB + i) * 8 + lrow;
    const int c = pch ^ ((r >> 1) & 7);
    const int64_t row = (int64_t)tm * BM + r;
    ob[i] = ((r < BM && row < M) ? (uint32_t)(row * K + c * 16) : kBig) - 1024u * (uint32_t)(i % 4);
  }
  // Scale copy (waves 0 and 1): lane l brings the 16 bytes of rows 4 l ..
  // 4 l + 3 of the tile from panel ks (offset ks * rows * 4 bytes, added per
  // step). Bytes of rows past the tile's owned rows or past N / M belong to
  // rows whose outputs are not stored (or read as zero past the array).
  const bool has_s = wid < 2;
  const uint32_t os = wid == 0 ? (uint32_t)(((int64_t)tn * p.rn + 4 * lane) * 4)
                               : (uint32_t)(((int64_t)tm * BM + 4 * lane) * 4);
  const int64_t spanel = wid == 0 ? N * 4 : M * 4;  // bytes per scale panel
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t la0 = lds0 + (uint32_t)(wid * NA) * 1024u;
  const uint32_t lb0 = lds0 + (uint32_t)(IA + wid * NB) * 1024u;
  const uint32_t ls0 = lds0 + (uint32_t)CODES + (uint32_t)(wid == 0 ? 0 : 1024);

  auto issue_group = [&](int g, int slot, int ks) {
    const int soff = ks * 128;
    const uint32_t so = (uint32_t)(slot * STAGE);
    const bool isA = g < GA;
    const int i0 = (isA ? g : g - GA) * 4;
    const uint32_t base = (isA ? la0 : lb0) + so + (uint32_t)i0 * 1024u;
    uint32_t vo[4];
    const int cnt = isA ? (NA - i0 < 4 ? NA - i0 : 4) : (NB - i0 < 4 ? NB - i0 : 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) vo[e] = isA ? oa[(i0 + e) < NA ? i0 + e : 0] : ob[(i0 + e) < NB ? i0 + e : 0];
    if (cnt == 4) mx_dma16<4>(base, vo, isA ? rw : rx, soff);
    else if (cnt == 3) mx_dma16<3>(base, vo, isA ? rw : rx, soff);
    else if (cnt == 2) mx_dma16<2>(base, vo, isA ? rw : rx, soff);
    else mx_dma16<1>(base, vo, isA ? rw : rx, soff);
  };
  auto issue_all = [&](int slot, int ks) {
#pragma unroll
    for (int g = 0; g < GA + GB; ++g) issue_group(g, slot, ks);
    if (has_s) {
      const uint32_t v[1] = {os};
      mx_dma16<1>(ls0 + (uint32_t)(slot * STAGE), v, wid == 0 ? rsw : rsx, (int)(ks * spanel));
    }
  };

  // MFMA operand reads: lane (row lr = l % T, group g = l / T) reads, for
  // sub-step h, chunks KI h / 16 + g and that + KI / 32 of its row and
  // scale byte KI h / 32 + g.
  const int lr = lane % T, lg = lane / T;
  const int sl = (lr >> 1) & 7;  // swizzle of rows lr (+ multiples of T)
  int x0[NKK], x1[NKK];
#pragma unroll
  for (int h = 0; h < NKK; ++h) {
    const int c0 = KI * h / 16 + lg;
    x0[h] = (c0 ^ sl) << 4;
    x1[h] = ((c0 + KI / 32) ^ sl) << 4;
  }
  const int rA = wn * WTN + lr, rB = wm * WTM + lr;

  acc_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = acc_t{};

  auto operand = [](const uint8_t* row, int o0, int o1) -> v8i {
    const uint4 u0 = *reinterpret_cast<const uint4*>(row + o0);
    const uint4 u1 = *reinterpret_cast<const uint4*>(row + o1);
    return v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
  };

  const int nk = p.nks;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue_all(s, s);
  int cs = 0, is = S - 1;
  for (int it = 0; it < nk; ++it) {
    if (has_s) mx_wait_stages<NI + 1, S - 2>(nk - 1 - it);
    else mx_wait_stages<NI, S - 2>(nk - 1 - it);
    __syncthreads();
    const uint8_t* st = smem + cs * STAGE;
#pragma unroll
    for (int h = 0; h < NKK; ++h) {
      v8i a[FN], bb[FM];
      int ea[FN], eb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        a[i] = operand(st + (rA + T * i) * 128, x0[h], x1[h]);
        ea[i] = st[CODES + (rA + T * i) * 4 + KI * h / 32 + lg];
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        bb[j] = operand(st + IA * 1024 + (rB + T * j) * 128, x0[h], x1[h]);
        eb[j] = st[CODES + 1024 + (rB + T * j) * 4 + KI * h / 32 + lg];
      }
      if (h == 0 && it + S - 1 < nk) issue_all(is, it + S - 1);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::run(a[i], bb[j], acc[i][j], ea[i], eb[j]);
    }
    cs = cs + 1 == S ? 0 : cs + 1;
    is = is + 1 == S ? 0 : is + 1;
  }

  // bf16 outputs go through the idle ring (every wave is past its last K
  // step and every copy has landed) so each lane stores 16 contiguous bytes
  // of a token's row; raw fp32 outputs and row strides that are not a
  // multiple of 8 take the direct stores below.
  constexpr int LDT = BN + 4;  // staged row stride in bf16 (8 bytes of padding)
  constexpr int CHF = (S * STAGE) / (LDT * 2);           // tokens that fit the ring
  constexpr int CH0 = CHF >= BM ? BM : CHF / WTM * WTM;  // chunk: whole wave tiles
  if constexpr (CH0 >= WTM) {
    if (!p.out_raw && (p.ldy & 7) == 0) {
      mx_store_staged<T, BN, BM, WN, WM, LDT, CH0>(p, acc, smem, tn, tm, wn, wm, lane, tid);
      return;
    }
  }

  // Register r of lane l: weight row 8 (r / 4) + 4 (l / T) + r % 4 of the
  // fragment, token l % T (for T = 16 only r < 4 exist).
  constexpr int NR = T == 16 ? 4 : 16;
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = (int64_t)tm * BM + wm * WTM + T * j + lr;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        const int nl = wn * WTN + T * i + 8 * q + 4 * lg;  // local weight row of register 4 q
        const int64_t n = (int64_t)tn * p.rn + nl;
        if (nl >= p.rn || n >= N) continue;
        // four consecutive outputs of one token: one 8- or 16-byte store
        // when they are all inside N and the row stride keeps it aligned
        const bool full4 = n + 3 < N && (p.ldy & 3) == 0;
        if (p.out_raw) {
          float* y = static_cast<float*>(p.Y) + m * p.ldy + n;
          if (full4) {
            *reinterpret_cast<float4*>(y) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                        acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) y[r] = acc[i][j][4 * q + r];
          }
        } else {
          uint32_t bb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) bb[r] = f32_to_bf16_rne(acc[i][j][4 * q + r]);
          uint16_t* y = static_cast<uint16_t*>(p.Y) + m * p.ldy + n;
          if (full4) {
            *reinterpret_cast<uint2*>(y) = make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) y[r] = (uint16_t)bb[r];
          }
        }
      }
    }
}

constexpr int kCUs = 256;  // MI355X compute units

template <int T, int BN, int BM, int WN, int WM, int S>
hipError_t launch_mx_dma(const MxDmaParams& p0, int rows, hipStream_t st) {
  MxDmaParams p = p0;
  p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.nks = (int)(p.K >> 7);
  // Rows per tile: shrink (to a multiple of 8, at least half the height)
  // so the blocks fill whole rounds of the CUs, unless a row count is given.
  if (rows <= 0) {
    const int64_t full = ((p.N + BN - 1) / BN) * p.tiles_m;
    const int64_t per = kCUs * ((full + kCUs - 1) / kCUs);
    const int64_t want = 8 * ((p.N * p.tiles_m + 8 * per - 1) / (8 * per));
    rows = (want >= BN / 2 && want < BN) ? (int)want : BN;
  }
  p.rn = rows;
  const int64_t tiles_n = (p.N + rows - 1) / rows;
  hipLaunchKernelGGL((mx_dma_kernel<T, BN, BM, WN, WM, S>), dim3((unsigned)(tiles_n * p.tiles_m)),
                     dim3(64 * WN * WM), 0, st, p);
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
  MxDmaParams p{static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
                M, N, K, Y, ldy, out_raw, 0, 0, 0};
  // Up to 32 tokens the product is a weight stream: 128-row tiles of 32
  // tokens (16 x 16 fragments), rows balanced over the CUs; above, 8-wave
  // 192 x 128 tiles (two waves per SIMD, each a 96 x 32 wave tile of three
  // 32 x 32 fragments, two MFMA sub-steps per K step), as for the
  // per-channel 256-token GEMM.
  if (M <= 32) return launch_mx_dma<16, 128, 32, 8, 1, 4>(p, 0, st);
  return launch_mx_dma<32, 192, 128, 2, 4, 3>(p, 192, st);
}

}  // namespace qr
