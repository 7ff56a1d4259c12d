// qr_linear_fused_noalloc: the per-linear call for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). It is qr_linear_fused with its workspace (split-K
// partial sums, then the activation codes and scales) in a fixed device
// array owned by the library instead of caller memory.
//
// The array lives in this code object: every GPU the library runs on holds
// its own copy, at its own device address, until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory, so its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever handed to kernels.
#include <mutex>

#include "qr_internal.h"
#include "qurl_w8a8.h"

namespace {

constexpr size_t kScratchBytes = (size_t)48 << 20;  // 48 MiB
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

extern "C" int qr_linear_fused_noalloc(const void* X, int64_t ldx, float act_mult, const void* Wq,
                                       const float* scale_w, int64_t M, int64_t N, int64_t K,
                                       int qt, void* Y, int64_t ldy, void* stream) {
  const char* fn = "qr_linear_fused_noalloc";
  // Shape errors first, with qr_linear_fused's own messages (it validates
  // before anything is enqueued and needs no workspace when M or N is 0).
  const size_t need = qr_workspace_size("qr_linear_fused", M, N, K, qt);
  if (need == (size_t)-1 || need == 0)
    return qr_linear_fused(X, ldx, act_mult, Wq, scale_w, M, N, K, qt, Y, ldy, nullptr, 0, stream);
  if (need > kScratchBytes)
    return qr::set_error(QR_ERR_WORKSPACE,
                         "qr_linear_fused_noalloc: this shape needs %zu bytes of scratch, more "
                         "than the library's fixed %zu",
                         need, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qr::hip_error(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return qr::set_error(QR_ERR_UNSUPPORTED, "%s: device %d beyond the %d supported", fn, dev,
                         kMaxDevices);
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_err[dev] != hipSuccess) return qr::hip_error(g_err[dev], fn);
  return qr_linear_fused(X, ldx, act_mult, Wq, scale_w, M, N, K, qt, Y, ldy, g_ptr[dev],
                         kScratchBytes, stream);
}
