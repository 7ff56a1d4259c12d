// Small-token linear for gfx950: the per-token quantization of the bf16
// input, the W8A8 product and the bf16 epilogue in one launch, for decode
// steps of a few tokens (M <= kSmallMaxM).
//
// The rollout linear of the QuRL paper notes ("Loss / training strategy":
// token-wise activation and channel-wise weight scales, INT8 or FP8;
// "Method > System integration": INT8/FP8 matrix multiplication in the
// rollout engine).
//
// Design (why a second kernel family): at one to four tokens the linear is a
// weight stream, and the general GEMM pays for things that do not stream
// weights: a separate quantizer launch for its input, and, on narrow layers,
// split K with a second kernel that adds the partial sums. Here
//  * one block owns 16 * RF output channels and the whole K. In every block
//    waves 0..QW-1 (QW = 1 to 4, one per 4096 input elements) quantize the
//    M token rows into an LDS panel [M][KP] (absmax over K, then the codes,
//    with the arithmetic of the per-token quantizer kernel: the same
//    helpers, so the codes and scales are the same bits) while the other
//    NSW = 8 - QW waves start streaming weights; the rows are a few to tens
//    of KB and come from L2 after the first block;
//  * the streaming waves split K instead of the blocks: wave w takes the
//    128-byte K chunks c = w - QW, w - QW + NSW, ...; each lane loads 16-byte
//    pieces of whole 128-byte weight lines into registers, PD chunks ahead,
//    which a per-wave LDS stage turns into the MFMA A operand (no barrier in
//    the loop), and reads the matching bytes of its token's codes from the
//    panel (the B operand; lanes of tokens >= M feed zeros). A and B use the
//    same K order inside an instruction, so the dot product is the plain one;
//  * the waves' partial sums meet in LDS and are added in wave order (FP8
//    sums are deterministic), then the GEMM epilogue
//    y = bf16_rne(fl32(fl32(fl32(acc) * sx[m]) * sw[n])) with
//    sx[m] = fl32(t_m * act_mult).
// No codes or partial sums go to memory and there is no second kernel.
#include <type_traits>

#include "qr_device.h"
#include "qr_small_m.h"

namespace qr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kNW = 8;                      // waves per block
constexpr int kSmallMaxQW = 4;              // waves that quantize the token rows, at most
constexpr int kBufWord3 = 0x00020000;       // raw buffer resource, 32-bit format, no swizzle
constexpr uint32_t kOOB = 0x80000000u;      // a buffer offset past every code matrix: reads 0
constexpr int kWeightNT = 2;                // cache policy of the weight loads: non-temporal

struct SmallParams {
  const uint16_t* X;
  int64_t ldx;
  float act_mult;
  const uint8_t* Wq;
  const float* sw;
  int M, N, K, KP;  // KP: panel row stride, K rounded up to 128
  uint16_t* Y;
  int64_t ldy;
};

// Weight loads: each wave instruction reads whole 128-byte lines (lane l
// takes 16-byte piece l % 8 of row l / 8 of an 8-row group), two per 16-row
// fragment; loads of 16 rows x 64 bytes, which the MFMA's lane layout would
// give directly, cost a quarter more time at the same bytes (each touches 16
// lines instead of 8). The rows reach the MFMA layout through a per-wave
// LDS stage. Chunks past the wave's last one (c >= nch) are issued as
// out-of-range loads (zeros, no memory traffic), so every step issues the
// same number of loads and the compiler's counted waits stay exact. Every
// weight line is read once, so the loads carry the non-temporal hint
// (measured 4-7% faster on the 7B-shaped linears at one and two tokens).
template <int RF>
__device__ __forceinline__ void load_chunk(v4u (&w)[RF][2], __amdgpu_buffer_rsrc_t rw,
                                           const uint32_t (&rowoff)[RF][2], int pl, int K, int c) {
  const int k0 = c * 128 + pl;
#pragma unroll
  for (int f = 0; f < RF; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t o = k0 < K ? rowoff[f][h] + (uint32_t)k0 : kOOB;
      w[f][h] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)o, 0, kWeightNT));
    }
}

// XOR swizzle of the 16-byte pieces of a 128-byte stage row: the MFMA reads
// put 16 rows at one logical piece; (r >> 1) & 7 spreads them over the banks.
__device__ __forceinline__ int stage_piece(int r, int p) { return p ^ ((r >> 1) & 7); }

template <int QT, int RF, int PD>
__global__ __launch_bounds__(kNW * 64) void small_m_linear_kernel(const SmallParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];  // panel, then partial sums
  __shared__ float tsh[kSmallMaxM];
  using acc_t = typename std::conditional<QT == kQInt8, v4i, v4f>::type;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.M, N = p.N, K = p.K, KP = p.KP;
  const int n0 = blockIdx.x * (16 * RF);
  const int nch = (K + 127) >> 7;
  // QW waves quantize the token rows (one per 4096 elements, at most
  // kSmallMaxQW); the other NSW stream the weights: wave w >= QW takes the
  // chunks c = w - QW + NSW i.
  const int QW = (int)min((int64_t)kSmallMaxQW, ((int64_t)M * K + 4095) / 4096);
  const int NSW = kNW - QW;
  const int nmine = (wave >= QW && wave - QW < nch) ? (nch - 1 - (wave - QW)) / NSW + 1 : 0;
  const int kl = 16 * (lane >> 4);  // MFMA layout: K bytes [kl, +16) and [64 + kl, +16) of a chunk

  // Weight rows of this lane's loads (row lane / 8 of each 8-row group);
  // rows past N read 0.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.Wq, (short)0, (int)((uint32_t)N * (uint32_t)K), kBufWord3);
  const int pl = 16 * (lane & 7);  // this lane's 16-byte piece of a line
  uint32_t rowoff[RF][2];
#pragma unroll
  for (int f = 0; f < RF; ++f)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = n0 + 16 * f + 8 * h + (lane >> 3);
      rowoff[f][h] = row < N ? (uint32_t)row * (uint32_t)K : kOOB;
    }
  // Per-wave stage: RF fragments of 16 rows x 128 bytes.
  __shared__ __attribute__((aligned(16))) uint8_t stage[kNW][RF][2048];
  uint8_t* stw = &stage[wave][0][0];
  int wr_off[2], rd_off[2];  // byte offsets inside one fragment
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + (lane >> 3);
    wr_off[h] = r * 128 + 16 * stage_piece(r, lane & 7);
    const int rr = lane & 15;
    rd_off[h] = rr * 128 + 16 * stage_piece(rr, 4 * h + (lane >> 4));
  }

  // The weight scales of this thread's outputs (read in the epilogue).
  constexpr int NOUT = (RF * 256 + kNW * 64 - 1) / (kNW * 64);
  float swv[NOUT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const int q = tid + o * kNW * 64;
    const int n = n0 + 16 * (q >> 8) + 4 * ((q & 63) >> 4) + ((q >> 6) & 3);
    swv[o] = (q < RF * 256 && n < N) ? p.sw[n] : 0.0f;
  }

  // Waves 0..Q-1 quantize the token rows while the others start the weight
  // stream (Q = 1 to 4 by the size of the rows). The rows go to LDS first
  // ([M][K] bf16, by LDS-DMA from wave 0, before any weight load: the CU's
  // memory pipeline serves requests in issue order, so rows requested after
  // the weights would wait for them; measured 4-10 us). A wave that has
  // issued a few chunks of weight loads cannot issue further instructions
  // until most of them are served, so the quantizing waves issue no weight
  // loads. The quantizing waves meet through LDS flags and counters (bounded
  // spins): rows landed, partial maxima written, codes written.
  const int nc8 = K >> 3;      // 16-byte chunks per token row
  const int nq = M * nc8;      // chunk q = m * nc8 + c at LDS byte 16 q
  uint8_t* xs = dsm;
  uint8_t* panel = dsm + small_m_rows_bytes(M, K);
  if (wave == 0) {
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.X, (short)0, (int)((uint32_t)(M - 1) * (uint32_t)p.ldx * 2u + (uint32_t)K * 2u),
        kBufWord3);
    const uint32_t xs0 = (uint32_t)(uintptr_t)xs;
    for (int j = 0; 64 * j < nq; ++j) {
      const int q = 64 * j + lane;
      uint32_t off = kOOB;
      if (q < nq) {
        const int m = q / nc8;
        off = (uint32_t)m * (uint32_t)p.ldx * 2u + (uint32_t)(q - m * nc8) * 16u;
      }
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(xs0 + 1024u * (uint32_t)j);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      // one wave instruction: 64 lanes x 16 bytes to LDS at M0 + 16 lane
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   : : "s"(m0), "v"(off), "s"(rx) : "memory", "m0");
#pragma clang diagnostic pop
    }
  }
  // [0] rows landed, [1] partial maxima written, [2] codes written
  __shared__ uint32_t flags[3];
  __shared__ float tpart[kSmallMaxQW][kSmallMaxM];
  if (tid < 3) flags[tid] = 0u;
  __syncthreads();  // orders the row loads before any weight load; waits for no memory
  auto spin_until = [&](int k, uint32_t v) {
    for (int it = 0; it < (1 << 22); ++it) {
      if (__hip_atomic_load(&flags[k], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= v) break;
      __builtin_amdgcn_s_sleep(1);
    }
  };

  acc_t acc[RF];
#pragma unroll
  for (int f = 0; f < RF; ++f) acc[f] = acc_t{};
  if (wave < QW) {
    if (wave == 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the rows are in LDS
      __hip_atomic_store(&flags[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      spin_until(0, 1u);
    }
    // Per-token absmax over the whole row, t = absmax / Q: this wave's
    // chunks c = 64 wave + lane + 64 QW i, then the waves' maxima.
#pragma unroll
    for (int m = 0; m < kSmallMaxM; ++m) {
      float a = 0.0f;
      if (m < M)
        for (int c = 64 * wave + lane; c < nc8; c += 64 * QW)
          a = fmaxf(a, absmax8_bf16(*reinterpret_cast<const uint4*>(xs + 16 * (m * nc8 + c))));
      a = wave_max(a);
      if (lane == 0) tpart[wave][m] = a;
    }
    if (lane == 0) __hip_atomic_fetch_add(&flags[1], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    spin_until(1, (uint32_t)QW);
    float t[kSmallMaxM];
#pragma unroll
    for (int m = 0; m < kSmallMaxM; ++m) {
      float a = tpart[0][m];
      for (int v = 1; v < QW; ++v) a = fmaxf(a, tpart[v][m]);
      t[m] = a / qmax<QT>();
      if (wave == 0 && lane == m) tsh[m] = t[m];
    }
    // Codes into the panel; the pad [K, KP) of each row holds zeros.
#pragma unroll
    for (int m = 0; m < kSmallMaxM; ++m) {
      if (m < M) {
        const float tm = t[m];
        for (int c = 64 * wave + lane; c < (KP >> 3); c += 64 * QW) {
          uint2 v = make_uint2(0u, 0u);
          if (c < nc8 && tm != 0.0f)
            v = codes8_bf16<QT>(*reinterpret_cast<const uint4*>(xs + 16 * (m * nc8 + c)), tm);
          *reinterpret_cast<uint2*>(panel + m * KP + c * 8) = v;
        }
      }
    }
    if (lane == 0) __hip_atomic_fetch_add(&flags[2], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    v4u w[PD][RF][2];
#pragma unroll
    for (int u = 0; u < PD; ++u) load_chunk<RF>(w[u], rw, rowoff, pl, K, wave - QW + u * NSW);
    // Wait for the panel. Every quantizing wave reaches its increment on
    // every path; the bound only keeps a wave from spinning forever if that
    // were ever broken.
    spin_until(2, (uint32_t)QW);

    // K loop: no barriers. Full rounds of PD chunks issue the same loads every
    // step, so the compiler's counted waits keep PD - 1 chunks in flight; the
    // last, partial round only consumes what is already loaded.
    const int tok = lane & 15;
    const bool tok_ok = tok < M;
    const uint8_t* prow = panel + (tok_ok ? tok : 0) * KP + kl;
    auto step = [&](const v4u (&wc)[RF][2], int c) {
      v4u b0 = v4u{0u, 0u, 0u, 0u}, b1 = v4u{0u, 0u, 0u, 0u};
      if (tok_ok) {
        b0 = *reinterpret_cast<const v4u*>(prow + c * 128);
        b1 = *reinterpret_cast<const v4u*>(prow + c * 128 + 64);
      }
      // whole lines into the stage, back out in the MFMA layout (one wave's
      // LDS accesses run in order: no wait between them)
#pragma unroll
      for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<v4u*>(stw + f * 2048 + wr_off[h]) = wc[f][h];
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        const v4u a0 = *reinterpret_cast<const v4u*>(stw + f * 2048 + rd_off[0]);
        const v4u a1 = *reinterpret_cast<const v4u*>(stw + f * 2048 + rd_off[1]);
        if constexpr (QT == kQInt8) {
          acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a0),
                                                         __builtin_bit_cast(v4i, b0), acc[f], 0, 0, 0);
          acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a1),
                                                         __builtin_bit_cast(v4i, b1), acc[f], 0, 0, 0);
        } else {
          const v8i a8 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                          (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          const v8i b8 = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                          (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          // format 0 = FP8 E4M3 for both operands; scale byte 127 = 2^0
          acc[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[f], 0, 0, 0, 127, 0, 127);
        }
      }
    };
    int i = 0;
    for (; i + PD <= nmine; i += PD) {
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        step(w[u], wave - QW + (i + u) * NSW);
        load_chunk<RF>(w[u], rw, rowoff, pl, K, wave - QW + (i + u + PD) * NSW);
      }
    }
#pragma unroll
    for (int u = 0; u < PD; ++u)
      if (i + u < nmine) step(w[u], wave - QW + (i + u) * NSW);
  }

  // Partial sums of the waves through LDS (the panel is dead after this
  // barrier), added in wave order. Register r of lane l of a 16x16 result is
  // output channel n0 + 16 f + 4 (l / 16) + r and token l % 16.
  __syncthreads();
  uint32_t* red = reinterpret_cast<uint32_t*>(dsm);
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const acc_t a = acc[f];
    uint32_t* dst = red + (wave * RF + f) * 256 + lane;
    if constexpr (QT == kQInt8) {
      dst[0] = (uint32_t)a.x;
      dst[64] = (uint32_t)a.y;
      dst[128] = (uint32_t)a.z;
      dst[192] = (uint32_t)a.w;
    } else {
      dst[0] = __float_as_uint(a.x);
      dst[64] = __float_as_uint(a.y);
      dst[128] = __float_as_uint(a.z);
      dst[192] = __float_as_uint(a.w);
    }
  }
  __syncthreads();
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const int q = tid + o * kNW * 64;
    if (q >= RF * 256) break;
    const int f = q >> 8, r = (q >> 6) & 3, l = q & 63;
    const int j = l & 15;
    const int n = n0 + 16 * f + 4 * (l >> 4) + r;
    if (j < M && n < N) {
      float a;
      if constexpr (QT == kQInt8) {
        int s = 0;
#pragma unroll
        for (int v = 0; v < kNW; ++v) s += (int)red[((v * RF + f) * 4 + r) * 64 + l];
        a = (float)s;
      } else {
        a = 0.0f;
#pragma unroll
        for (int v = 0; v < kNW; ++v) a += __uint_as_float(red[((v * RF + f) * 4 + r) * 64 + l]);
      }
      const float sx = tsh[j] * p.act_mult;
      p.Y[(int64_t)j * p.ldy + n] = (uint16_t)epi_bf16(a, sx, swv[o]);
    }
  }
}

// Chunks kept in flight per wave for RF fragments (registers: 8 RF PD; some
// FP8 kernels keep one chunk fewer, to stay within their registers).
constexpr int pd_for(int qt, int rf) {
  return rf == 1 ? 8 : rf == 2 ? (qt == kQFp8 ? 5 : 6) : rf == 3 ? (qt == kQFp8 ? 3 : 4)
         : (rf == 5 && qt == kQFp8) ? 2 : 3;
}

template <int QT, int RF>
hipError_t launch_rf(const SmallParams& p, hipStream_t st) {
  const size_t lds = small_m_lds_bytes(p.M, p.K, RF);
  const unsigned blocks = (unsigned)((p.N + 16 * RF - 1) / (16 * RF));
  hipLaunchKernelGGL((small_m_linear_kernel<QT, RF, pd_for(QT, RF)>), dim3(blocks), dim3(kNW * 64), lds,
                     st, p);
  return hipGetLastError();
}

template <int QT>
hipError_t launch_qt(const SmallParams& p, int rf, hipStream_t st) {
  switch (rf) {
    case 1: return launch_rf<QT, 1>(p, st);
    case 2: return launch_rf<QT, 2>(p, st);
    case 3: return launch_rf<QT, 3>(p, st);
    case 4: return launch_rf<QT, 4>(p, st);
    default: return launch_rf<QT, 5>(p, st);
  }
}

}  // namespace

size_t small_m_lds_bytes(int64_t M, int64_t K, int rf) {
  const size_t rows_panel = small_m_rows_bytes(M, K) + (size_t)M * (size_t)(((K + 127) / 128) * 128);
  const size_t red = (size_t)kNW * rf * 4 * 64 * 4;
  return rows_panel > red ? rows_panel : red;
}

bool small_m_ok(int64_t M, int64_t N, int64_t K, int64_t ldx) {
  // (the rows' buffer resource spans (M - 1) ldx + K bf16 values: 31 bits)
  return M >= 1 && M <= kSmallMaxM && N >= 1 && K >= 16 && K % 16 == 0 &&
         M * K <= kSmallMaxMK && ((M - 1) * ldx + K) * 2 < ((int64_t)1 << 31) - ((int64_t)1 << 16);
}

bool small_m_auto(int64_t M, int64_t N, int64_t K, int64_t ldx) {
  // Measured on MI355X (graph-replayed, against the quantizer and GEMM
  // launches): faster up to M K = 8192 (the 7B-shaped QKV, O, gate and up
  // at 1 and 2 tokens: 9.0 / 8.2 / 16.0 us against 12.0 / 10.7 / 17.9 us at
  // one token); equal for the 7B down projection at one token (K = 18944);
  // slower at 4 tokens of K = 3584.
  return small_m_ok(M, N, K, ldx) && M * K <= 8192;
}

int small_m_rf(int64_t N, int force_rf) {
  if (force_rf >= 1 && force_rf <= kSmallMaxRF) return force_rf;
  // The fewest 16-row fragments per block that keep the grid within one
  // block per CU (measured: 4608 rows on 32-row blocks 9.0 us, on 16-row
  // blocks 11.5 us), at most five.
  for (int rf = 1; rf < kSmallMaxRF; ++rf)
    if ((N + 16 * rf - 1) / (16 * rf) <= 256) return rf;
  return kSmallMaxRF;
}

hipError_t launch_small_m_linear(const void* X, int64_t ldx, float act_mult, const void* Wq,
                                 const float* scale_w, int64_t M, int64_t N, int64_t K, int qt,
                                 void* Y, int64_t ldy, int rf, hipStream_t st) {
  SmallParams p;
  p.X = static_cast<const uint16_t*>(X);
  p.ldx = ldx;
  p.act_mult = act_mult;
  p.Wq = static_cast<const uint8_t*>(Wq);
  p.sw = scale_w;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.KP = (int)(((K + 127) / 128) * 128);
  p.Y = static_cast<uint16_t*>(Y);
  p.ldy = ldy;
  return qt == kQInt8 ? launch_qt<kQInt8>(p, rf, st) : launch_qt<kQFp8>(p, rf, st);
}

}  // namespace qr
