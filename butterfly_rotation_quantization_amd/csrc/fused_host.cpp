// Host dispatch of the fast paths (MFMA tile kernels) -- not yet enabled: every call goes through
// the generic tile pass.
#include "fused.h"

namespace brq {

hipError_t fused_prepare(Plan&) { return hipSuccess; }
void fused_release(Plan&) {}

bool fused_rotate_supported(const Plan*, const Plan*, int, int, int64_t, int64_t, int64_t, int64_t,
                            const void*, const void*) {
  return false;
}
hipError_t fused_rotate(const Plan*, const Plan*, const void*, int, int64_t, void*, int, int64_t,
                        int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

bool fused_rqp_supported(const Plan*, const Plan*, int, int64_t, int64_t, int64_t, const void*,
                         const brq_quant*) {
  return false;
}
brq_status fused_rqp(const Plan*, const Plan*, const void*, int, int64_t, int64_t, int64_t,
                     const brq_quant*, uint8_t*, void*, void*, size_t, hipStream_t) {
  return BRQ_ERR_UNSUPPORTED;
}

}  // namespace brq
