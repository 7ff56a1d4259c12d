// Measurement helpers: the peaks the chip actually reaches, so that the
// GEMMs' roofline fractions can be given against measured peaks as well as
// the datasheet ones.
//
//  * read_probe_kernel streams a buffer once with 16-byte non-temporal loads
//    (eight in flight per thread) and keeps one XOR word per block, so the
//    loads cannot be removed. Bytes / time = the HBM read rate (for a buffer
//    well past the 256 MB Infinity Cache).
//  * copy_stream_probe_kernel replays the operand copies of one LDS-DMA GEMM
//    tiling (the same blocks, copies, ring, waits and barriers) with no
//    fragment reads and no MFMAs: the time the copy pipeline alone needs
//    for that tiling, against which the GEMM's own time can be read. Its
//    variants (padded row strides, weights stored as K panels, no barrier
//    per K step) measure what each of those would change in the copies.
//  * mfma_probe_kernel runs rounds of eight independent dense 8-bit MFMAs
//    (INT8 32x32x32 or FP8 32x32x64, the shapes the GEMMs use) per wave on
//    register operands. Wave 0 of each block reads the shader-clock counter
//    and the constant-rate wall clock at its start and end, so the host can
//    tell the shader clock the matrix cores ran at.
#include "qr_copy.h"
#include "qr_internal.h"

namespace qr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Block b reads its own contiguous 1/grid of the buffer; every thread keeps
// eight 16-byte non-temporal loads in flight (a wave reads 1 KB contiguous
// per load). Measured on MI355X over 4 GiB: 7.0 TB/s, against 6.1-6.3 TB/s
// with plain loads and 5.7 TB/s with a grid-strided loop of four.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  constexpr int U = 8, NT = 256;
  __shared__ uint32_t red[NT];
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t x = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * NT < b1; i += U * NT) {
    v4u r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      r[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(&src[i + u * NT]));
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (; i < b1; i += NT) {
    const uint4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  red[threadIdx.x] = x;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

template <int QT>
__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, uint32_t* __restrict__ sink,
                                                         uint64_t* __restrict__ ticks) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint64_t c0 = 0, w0 = 0;
  if (threadIdx.x == 0) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  uint32_t h = 0;
  if constexpr (QT == kQInt8) {
    const v4i a = {lane, lane + 1, lane + 2, lane + 3};
    const v4i b = {lane * 3, lane + 7, 5, lane};
    v16i acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) h ^= (uint32_t)acc[j][e];
  } else {
    // E4M3FN bytes 0x38 (1.0) and 0x30 (0.5): finite products, exact sums.
    const v8i a = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                   0x38383838, 0x38383838, 0x38383838, 0x38383838};
    const v8i b = {0x30303030, 0x30303030, 0x30303030, 0x30303030,
                   0x30303030, 0x30303030, 0x30303030, 0x30303030};
    v16f acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v16f{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) h ^= __float_as_uint(acc[j][e]);
  }
  for (int o = 32; o > 0; o >>= 1) h ^= (uint32_t)__shfl_xor((int)h, o, 64);
  if (lane == 0) sink[(int64_t)blockIdx.x * 8 + wave] = h;
  if (threadIdx.x == 0) {
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    ticks[4 * (int64_t)blockIdx.x + 0] = c0;
    ticks[4 * (int64_t)blockIdx.x + 1] = c1;
    ticks[4 * (int64_t)blockIdx.x + 2] = w0;
    ticks[4 * (int64_t)blockIdx.x + 3] = w1;
  }
}

// Block b (dealt to the XCDs round-robin and ordered token tile fastest, as
// the GEMM deals its blocks) copies weight rows [tn * rows, tn * rows + rows)
// and token rows [tm * BM, tm * BM + BM) over K in 128-byte steps into an
// S-slot LDS ring: wave w copies weight row blocks (1 KB = 8 rows) w * NA ..
// w * NA + NA - 1 and token row blocks w * NB .. w * NB + NB - 1 of every
// step, the lane owning physical chunk c of row r fetching logical chunk
// c ^ ((r >> 1) & 7); rows outside the tile or the matrix read as zero. Each
// wave waits for its own copies of a step, all meet at one barrier per step
// (SYNC; without it every wave runs ahead on its own waits alone), and the
// copies of step it + S - 1 are issued after it. Row r of the weights starts
// at byte r * ldw, K step k at k * kb within it (kb = 128; kb = 0 re-reads
// the first step's bytes at every step, so after the first step the operands
// come from L2); PANEL instead reads the weights as K panels, K step k of
// row r at byte (k * N + r) * 128 (k * kb / 128 panels in), so one step of a
// tile is one contiguous block. Token row r starts at r * ldx. Thread 0 then
// writes sink[b] = XOR of the first 16 bytes of the block's first weight row
// and of its first token row in the last K step, as they arrived in LDS.
template <int BN, int BM, int NW, int S, bool NTW, bool PANEL, bool SYNC>
__global__ __launch_bounds__(64 * NW, 1) void copy_stream_probe_kernel(
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, int64_t N, int64_t M, int64_t K,
    int64_t ldw, int64_t ldx, int rows, int tiles_m, int kb, uint32_t* __restrict__ sink) {
  constexpr int BK = 128, RB = 8, CPR = 8;
  constexpr int IA = BN / RB, IB = BM / RB;
  static_assert(IA % NW == 0 && IB % NW == 0, "row blocks per wave");
  constexpr int NA = IA / NW, NB = IB / NW, NI = NA + NB;
  static_assert(NA >= 1 && NA <= 4 && NB >= 1 && NB <= 4, "one M0 group per operand");
  constexpr int STAGE = (IA + IB) * 1024;
  static_assert(S >= 2 && S * STAGE <= 160 * 1024 && (S - 2) * NI <= 63, "ring");
  constexpr uint32_t kOOB = 0x80000000u;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int G = gridDim.x, G8 = G & ~7;
  int b = blockIdx.x;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  const int tm = b % tiles_m, tn = b / tiles_m;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nk = (int)(K / BK);
  const int64_t wbytes = PANEL ? (int64_t)nk * N * BK : N * ldw;
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)(uint32_t)wbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsx =
      __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)(uint32_t)(M * ldx), kBufWord3);
  const int lrow = lane / CPR, pch = lane % CPR;
  uint32_t oa[NA], ob[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = (wid * NA + i) * RB + lrow;
    const int c = pch ^ ((r >> 1) & 7);
    const int64_t row = (int64_t)tn * rows + r;
    oa[i] = ((r < rows && row < N) ? (uint32_t)(row * (PANEL ? (int64_t)BK : ldw) + c * 16) : kOOB) -
            1024u * (uint32_t)i;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = (wid * NB + i) * RB + lrow;
    const int c = pch ^ ((r >> 1) & 7);
    const int64_t row = (int64_t)tm * BM + r;
    ob[i] = ((row < M) ? (uint32_t)(row * ldx + c * 16) : kOOB) - 1024u * (uint32_t)i;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t la0 = lds0 + (uint32_t)(wid * NA) * 1024u;
  const uint32_t lb0 = lds0 + (uint32_t)(IA + wid * NB) * 1024u;
  auto issue = [&](int slot, int ks) {
    const int soff = ks * kb;
    const int soffw = PANEL ? (int)((int64_t)ks * N * kb) : soff;
    dma_group<NA, NTW>(la0 + (uint32_t)(slot * STAGE), oa, rsw, soffw);
    dma_group<NB, false>(lb0 + (uint32_t)(slot * STAGE), ob, rsx, soff);
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
  int is = S - 1;
  for (int it = 0; it < nk; ++it) {
    wait_stages<NI, S - 2>(nk - 1 - it);
    if constexpr (SYNC) __syncthreads();
    if (it + S - 1 < nk) issue(is, it + S - 1);
    is = is + 1 == S ? 0 : is + 1;
  }
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int last = (nk - 1) % S;
    const uint32_t* wa = reinterpret_cast<const uint32_t*>(smem + last * STAGE);
    const uint32_t* xa = reinterpret_cast<const uint32_t*>(smem + last * STAGE + IA * 1024);
    sink[b] = wa[0] ^ wa[1] ^ wa[2] ^ wa[3] ^ xa[0] ^ xa[1] ^ xa[2] ^ xa[3];
  }
}

template <int BN, int BM, int S, bool NTW>
hipError_t launch_copy_stream(dim3 grid, int flags, const uint8_t* w, const uint8_t* x, int64_t N,
                              int64_t M, int64_t K, int64_t ldw, int64_t ldx, int rows, int tiles_m,
                              uint32_t* sink, hipStream_t st) {
  const bool panel = (flags & 1) != 0, sync = (flags & 2) == 0;
  const int kb = (flags & 4) ? 0 : 128;
  if (panel && sync)
    hipLaunchKernelGGL((copy_stream_probe_kernel<BN, BM, 8, S, NTW, true, true>), grid, dim3(512), 0,
                       st, w, x, N, M, K, ldw, ldx, rows, tiles_m, kb, sink);
  else if (panel)
    hipLaunchKernelGGL((copy_stream_probe_kernel<BN, BM, 8, S, NTW, true, false>), grid, dim3(512), 0,
                       st, w, x, N, M, K, ldw, ldx, rows, tiles_m, kb, sink);
  else if (sync)
    hipLaunchKernelGGL((copy_stream_probe_kernel<BN, BM, 8, S, NTW, false, true>), grid, dim3(512), 0,
                       st, w, x, N, M, K, ldw, ldx, rows, tiles_m, kb, sink);
  else
    hipLaunchKernelGGL((copy_stream_probe_kernel<BN, BM, 8, S, NTW, false, false>), grid, dim3(512), 0,
                       st, w, x, N, M, K, ldw, ldx, rows, tiles_m, kb, sink);
  return hipGetLastError();
}

}  // namespace

unsigned read_probe_blocks() { return 1024; }

// Geometry of the GEMM tilings the copy-stream probe replays (tile index of
// the GEMM planner; the same ring depth, waves and hint on the weights).
bool copy_stream_probe_tile(int tile, int& bn, int& bm) {
  if (tile == 4) { bn = 256; bm = 256; return true; }
  if (tile == 8) { bn = 192; bm = 128; return true; }
  if (tile == 10) { bn = 192; bm = 256; return true; }
  return false;
}

hipError_t launch_copy_stream_probe(int tile, const void* W, const void* X, int64_t N, int64_t M,
                                    int64_t K, int64_t ldw, int64_t ldx, int rows, int flags,
                                    uint32_t* sink, hipStream_t st) {
  int bn = 0, bm = 0;
  if (!copy_stream_probe_tile(tile, bn, bm)) return hipErrorInvalidValue;
  const int64_t tiles_m = (M + bm - 1) / bm, tiles_n = (N + rows - 1) / rows;
  const dim3 grid((unsigned)(tiles_n * tiles_m));
  const uint8_t* w = static_cast<const uint8_t*>(W);
  const uint8_t* x = static_cast<const uint8_t*>(X);
  if (tile == 4)
    return launch_copy_stream<256, 256, 2, true>(grid, flags, w, x, N, M, K, ldw, ldx, rows,
                                                 (int)tiles_m, sink, st);
  if (tile == 10)
    return launch_copy_stream<192, 256, 2, true>(grid, flags, w, x, N, M, K, ldw, ldx, rows,
                                                 (int)tiles_m, sink, st);
  return launch_copy_stream<192, 128, 4, false>(grid, flags, w, x, N, M, K, ldw, ldx, rows,
                                                (int)tiles_m, sink, st);
}

hipError_t launch_read_probe(const void* buf, int64_t n16, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(read_probe_blocks()), dim3(256), 0, st,
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int qt, int blocks, int iters, uint32_t* sink, uint64_t* ticks,
                             hipStream_t st) {
  if (qt == kQInt8)
    hipLaunchKernelGGL(mfma_probe_kernel<kQInt8>, dim3(blocks), dim3(512), 0, st, iters, sink, ticks);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<kQFp8>, dim3(blocks), dim3(512), 0, st, iters, sink, ticks);
  return hipGetLastError();
}

}  // namespace qr
