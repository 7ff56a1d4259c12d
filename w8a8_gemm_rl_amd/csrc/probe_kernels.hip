// Measurement helpers: the peaks the chip actually reaches, so that the
// GEMMs' roofline fractions can be given against measured peaks as well as
// the datasheet ones.
//
//  * read_probe_kernel streams a buffer once with 16-byte non-temporal loads
//    (eight in flight per thread) and keeps one XOR word per block, so the
//    loads cannot be removed. Bytes / time = the HBM read rate (for a buffer
//    well past the 256 MB Infinity Cache).
//  * mfma_probe_kernel runs rounds of eight independent dense 8-bit MFMAs
//    (INT8 32x32x32 or FP8 32x32x64, the shapes the GEMMs use) per wave on
//    register operands. Wave 0 of each block reads the shader-clock counter
//    and the constant-rate wall clock at its start and end, so the host can
//    tell the shader clock the matrix cores ran at.
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

}  // namespace

unsigned read_probe_blocks() { return 1024; }

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
