// LDS-DMA copies shared by the GEMM kernels and the copy-stream probe.
//
// buffer_load_dwordx4 ... lds moves 64 x 16 bytes from global memory
// straight into LDS: lane l's 16 bytes land at M0 + offset + 16 * l, where
// the 12-bit instruction offset also advances the global address. A wave's
// copies go to consecutive 1 KB LDS blocks, so up to four share one M0 write
// (offsets 0, 1 KB, 2 KB, 3 KB; the per-lane global offsets are pre-biased by
// minus the instruction offset). Offsets past the buffer resource's
// num_records read as zero, which is how rows outside a matrix are copied.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

// Word 3 of a raw buffer resource on gfx9 parts: 32-bit data format, no
// swizzle; with stride 0 the bound check is offset < num_records.
constexpr int kBufWord3 = 0x00020000;

// NT: the non-temporal hint on the copies (data streamed once).
template <int CNT, bool NT>
__device__ __forceinline__ void dma_group(uint32_t lds_addr, const uint32_t* vo,
                                          __amdgpu_buffer_rsrc_t r, int soff) {
  static_assert(CNT >= 1 && CNT <= 4, "one M0 covers at most 4 KB of offsets");
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (CNT == 1 && !NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 : : "s"(lds_addr), "v"(vo[0]), "s"(r), "s"(soff) : "memory", "m0");
  else if constexpr (CNT == 1)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 : : "s"(lds_addr), "v"(vo[0]), "s"(r), "s"(soff) : "memory", "m0");
  else if constexpr (CNT == 2 && !NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds"
        : : "s"(lds_addr), "v"(vo[0]), "v"(vo[1]), "s"(r), "s"(soff) : "memory", "m0");
  else if constexpr (CNT == 2)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen nt lds\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 nt lds"
        : : "s"(lds_addr), "v"(vo[0]), "v"(vo[1]), "s"(r), "s"(soff) : "memory", "m0");
  else if constexpr (CNT == 3 && !NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %4, %5 offen lds\n\t"
        "buffer_load_dwordx4 %2, %4, %5 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %4, %5 offen offset:2048 lds"
        : : "s"(lds_addr), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "s"(r), "s"(soff)
        : "memory", "m0");
  else if constexpr (CNT == 3)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %4, %5 offen nt lds\n\t"
        "buffer_load_dwordx4 %2, %4, %5 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %3, %4, %5 offen offset:2048 nt lds"
        : : "s"(lds_addr), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "s"(r), "s"(soff)
        : "memory", "m0");
  else if constexpr (!NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
        "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
        : : "s"(lds_addr), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(r), "s"(soff)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %5, %6 offen nt lds\n\t"
        "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 nt lds\n\t"
        "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 nt lds"
        : : "s"(lds_addr), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(r), "s"(soff)
        : "memory", "m0");
#pragma clang diagnostic pop
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most min(ahead, A) stages of this wave's copies (NI
// instructions each) are still in flight; A = S - 2 is the most a ring of S
// slots ever has outstanding behind the step being consumed.
template <int NI, int A>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (A > 0) {
    if (ahead >= A) {
      wait_vm<A * NI>();
      return;
    }
    wait_stages<NI, A - 1>(ahead);
  } else {
    wait_vm<0>();
  }
}

}  // namespace qr
