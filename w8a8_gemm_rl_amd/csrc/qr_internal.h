// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qr_device.h"
#include "qr_gemm.h"
#include "qr_small_m.h"

namespace qr {

hipError_t launch_act_quant(const void* X, int64_t M, int64_t K, int64_t ldx, float act_mult,
                            int qt, void* Xq, float* scale_x, hipStream_t st);
hipError_t launch_weight_quant(const float* W, int64_t N, int64_t K, int64_t ldw, float s, int qt,
                               void* Wq, float* scale_w, float* Wsc, hipStream_t st);
hipError_t launch_fold_norm(float* gamma, float* beta, int64_t K, float s, hipStream_t st);
hipError_t launch_norm_quant(const void* H, int64_t M, int64_t K, int64_t ldh, int kind,
                             const float* gamma, const float* beta, float eps, int qt, void* Xq,
                             float* scale_x, hipStream_t st);
hipError_t launch_silu_mul_quant(const void* G, const void* U, int64_t M, int64_t N, int64_t ldg,
                                 int64_t ldu, float act_mult, int qt, void* Xq, float* scale_x,
                                 hipStream_t st);
hipError_t launch_mx_quant(const void* A, int64_t R, int64_t K, int64_t lda, int bf16,
                           void* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_mx_gemm(const void* Xq, const uint8_t* sx, const void* Wq, const uint8_t* sw,
                          int64_t M, int64_t N, int64_t K, int out_raw, void* Y, int64_t ldy,
                          hipStream_t st);
int64_t acr_blocks(int64_t n);
hipError_t launch_acr_tis(const float* logp, const float* lprox, const float* lbeh,
                          const float* adv, const uint8_t* mask, int64_t n, float eps, float C,
                          float* loss, float* grad, double* sums, double* part, hipStream_t st);
hipError_t launch_requant(const float* Wp, int64_t N, int64_t K, int64_t ldw, int qt, void* Wq,
                          float* scale_w, uint32_t* row_flips, hipStream_t st);

// Error reporting of the C ABI (qr_last_error): set the thread-local message
// and return `code`; hip_error maps a HIP error to QR_ERR_HIP / QR_ERR_NO_DEVICE.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_error(hipError_t e, const char* what);

unsigned read_probe_blocks();
hipError_t launch_read_probe(const void* buf, int64_t n16, uint32_t* sink, hipStream_t st);
bool copy_stream_probe_tile(int tile, int& bn, int& bm);
hipError_t launch_copy_stream_probe(int tile, const void* W, const void* X, int64_t N, int64_t M,
                                    int64_t K, int64_t ldw, int64_t ldx, int rows, int flags,
                                    uint32_t* sink, hipStream_t st);
hipError_t launch_mfma_probe(int qt, int blocks, int iters, uint32_t* sink, uint64_t* ticks,
                             hipStream_t st);

}  // namespace qr
