// Fast paths for common plan shapes (MFMA tile kernels).  Each entry point
// reports whether it covers a call; the generic tile pass handles the rest.
#pragma once

#include "brq_internal.h"

namespace brq {

// Per-plan device data of the fast paths (called at plan creation / destroy).
hipError_t fused_prepare(Plan& p);
void fused_release(Plan& p);

bool fused_rotate_supported(const Plan* U, const Plan* V, int xt, int yt, int64_t rows,
                            int64_t cols, int64_t ldx, int64_t ldy, const void* x, const void* y);
hipError_t fused_rotate(const Plan* U, const Plan* V, const void* x, int xt, int64_t ldx, void* y,
                        int yt, int64_t ldy, int64_t rows, int64_t cols, hipStream_t s);

bool fused_rqp_supported(const Plan* U, const Plan* V, int wt, int64_t m, int64_t n, int64_t ldw,
                         const void* w, const brq_quant* q);
brq_status fused_rqp(const Plan* U, const Plan* V, const void* w, int wt, int64_t m, int64_t n,
                     int64_t ldw, const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                     size_t ws_bytes, hipStream_t s);

}  // namespace brq
