// The decode linear without a caller workspace and without allocation, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops).  Its scratch -- the rotated activations, the split
// partial sums, Z and the rotations' intermediate -- lives in a file-scope
// device array of kScratchBytes, one copy per GPU for the life of the
// process.  The array's device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels: the array's name in host code is a host-side
// stand-in, not a device address.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "brq_internal.h"

namespace brq {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up on first use.
brq_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report_error(BRQ_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return report_error(BRQ_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress of the scratch array: %s",
               hipGetErrorString(e));
      return report_error(BRQ_ERR_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BRQ_OK;
}

}  // namespace
}  // namespace brq

extern "C" {

size_t brq_qlinear_noalloc_limit(void) { return brq::kScratchBytes; }

brq_status brq_qlinear_noalloc(const brq_plan* left, const brq_plan* right, const void* x,
                               int32_t xt, int64_t ldx, int64_t T, const uint8_t* codes,
                               const void* scales, const brq_quant* q, int64_t m, int64_t n,
                               void* y, int32_t yt, int64_t ldy, void* stream) {
  if (!q) return brq::report_error(BRQ_ERR_INVALID_ARGUMENT, "NULL quantizer");
  const size_t need = brq_qlinear_workspace_bytes(left, right, q, T, m, n);
  if (need > brq::kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "this call needs %zu bytes of scratch, more than the %zu bytes the no-allocation "
             "entry point holds per device; use brq_qlinear with a workspace",
             need, brq::kScratchBytes);
    return brq::report_error(BRQ_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  const brq_status st = brq::scratch_for_current_device(&ws);
  if (st != BRQ_OK) return st;
  return brq_qlinear(left, right, x, xt, ldx, T, codes, scales, q, m, n, y, yt, ldy, ws,
                     brq::kScratchBytes, stream);
}

}  // extern "C"
