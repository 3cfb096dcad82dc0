// HARP blocks from their parameters: B = Q(theta) G per group, Q a Givens
// rotation (b = 2) or the Cayley map (I - A)^{-1}(I + A) of a skew-symmetric
// A (b > 2), G the normalised Sylvester matrix or a given base mixer.
//
// One wavefront per block.  The b x 2b matrix [I - A | I + A] is reduced by
// Gauss-Jordan elimination in float64 (no pivoting: the symmetric part of
// I - A is I, so every pivot is at least 1 and the elimination is stable).
// Up to b = 32 each lane keeps one column in registers and the pivot column
// is broadcast lane to lane; above, the system sits in LDS and lane l owns
// columns l and l + 64.  The right half is then Q, and lane l forms entries
// l, l + 64, ... of Q G, rounded once to float32.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kHpThreads = 64;

struct HarpArgs {
  int b;               // radix, 2..64
  int np;              // parameters per block: 1 (b = 2) or b(b-1)/2
  int64_t ngroups;     // blocks to build
  const int8_t* theta; // [ngroups][np] int8
  float scale;         // theta = scale * q
  const float* base;   // G [b][b] row-major, or null: Sylvester / sqrt(b)
  float* out;          // [ngroups][b][b]
};

__host__ __device__ inline int harp_params(int b) { return b == 2 ? 1 : b * (b - 1) / 2; }
// Parameter index of A[i][j], i < j: the strict upper triangle, row-major.
__host__ __device__ inline int harp_pidx(int b, int i, int j) {
  return i * b - i * (i + 1) / 2 + (j - i - 1);
}
// LDS: the b x 2b system with a row pitch of 2b + 1 doubles, then b factors.
__host__ __device__ inline int harp_pitch(int b) { return 2 * b + 1; }
__host__ __device__ inline size_t harp_lds_bytes(int b) {
  return ((size_t)b * harp_pitch(b) + b) * sizeof(double);
}

hipError_t launch_harp(const HarpArgs& a, hipStream_t s);

// Several stages in one launch (3 <= b <= 32 each, the register kernel's
// range): workgroup w builds block w - first[j] of job j, first[j] <= w <
// first[j + 1].  The stages of a plan are independent, so one launch lets
// the few long radix-32 eliminations overlap the many short ones instead of
// running stage after stage.
constexpr int kHpMaxJobs = 16;
struct HarpBatch {
  int n;
  HarpArgs job[kHpMaxJobs];
  int64_t first[kHpMaxJobs + 1];
};
__host__ __device__ inline bool harp_batchable(int b) { return b >= 3 && b <= 32; }
hipError_t launch_harp_batch(const HarpBatch& a, hipStream_t s);

}  // namespace brq
