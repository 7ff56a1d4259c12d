// Host interface of the small-token linear (small_m_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qr {

// The small-token linear (quantization of the bf16 input, product and
// epilogue in one launch) for M <= kSmallMaxM token rows, M K <= kSmallMaxMK;
// it holds the bf16 rows and their codes ([M][K rounded up to 128]) in LDS.
constexpr int kSmallMaxM = 4;
constexpr int kSmallMaxRF = 5;
constexpr int64_t kSmallMaxMK = 20480;  // M K: bf16 rows and codes fit the LDS beside the stage
// LDS bytes of the bf16 token rows, rounded up to whole 1 KB LDS-DMA copies.
__host__ __device__ inline size_t small_m_rows_bytes(int64_t M, int64_t K) {
  return (size_t)(((M * K * 2 + 1023) / 1024) * 1024);
}
size_t small_m_lds_bytes(int64_t M, int64_t K, int rf);
bool small_m_ok(int64_t M, int64_t N, int64_t K, int64_t ldx);    // the kernel can run it
bool small_m_auto(int64_t M, int64_t N, int64_t K, int64_t ldx);  // and it is the faster path
int small_m_rf(int64_t N, int force_rf);
hipError_t launch_small_m_linear(const void* X, int64_t ldx, float act_mult, const void* Wq,
                                 const float* scale_w, int64_t M, int64_t N, int64_t K, int qt,
                                 void* Y, int64_t ldy, int rf, hipStream_t st);

}  // namespace qr
