// HARP block builder kernel (harp.h).
#include "harp.h"

namespace brq {
namespace {

__global__ __launch_bounds__(kHpThreads) void harp_kernel(HarpArgs a) {
  extern __shared__ double hp_lds[];
  const int b = a.b, P = harp_pitch(b), lane = threadIdx.x;
  double* m = hp_lds;            // [b][P]: columns 0..b-1 = I - A, b..2b-1 = I + A
  double* fac = hp_lds + b * P;  // column i of the current step
  const int64_t g = blockIdx.x;
  const int8_t* th = a.theta + g * a.np;
  const double sc = (double)a.scale;

  if (b == 2) {
    // Givens: Q = [[c, -s], [s, c]] into the right half
    if (lane == 0) {
      const double t = sc * (double)th[0];
      const double c = cos(t), s = sin(t);
      m[0 * P + 2] = c;
      m[0 * P + 3] = -s;
      m[1 * P + 2] = s;
      m[1 * P + 3] = c;
    }
  } else {
    for (int e = lane; e < b * b; e += kHpThreads) {
      const int i = e / b, j = e - i * b;
      double aij = 0.0;
      if (i < j) aij = sc * (double)th[harp_pidx(b, i, j)];
      else if (i > j) aij = -sc * (double)th[harp_pidx(b, j, i)];
      const double id = i == j ? 1.0 : 0.0;
      m[i * P + j] = id - aij;
      m[i * P + b + j] = id + aij;
    }
    for (int i = 0; i < b; ++i) {
      __syncthreads();  // the previous step's columns are written
      if (lane < b) fac[lane] = m[lane * P + i];
      __syncthreads();
      const double inv = 1.0 / fac[i];
      for (int c = lane; c < 2 * b; c += kHpThreads) {
        const double pc = m[i * P + c] * inv;
        for (int r = 0; r < b; ++r)
          if (r != i) m[r * P + c] = fma(-fac[r], pc, m[r * P + c]);
        m[i * P + c] = pc;
      }
    }
  }
  __syncthreads();

  // B = Q G, rounded once
  const double hs = 1.0 / sqrt((double)b);
  float* out = a.out + g * b * b;
  for (int e = lane; e < b * b; e += kHpThreads) {
    const int j = e / b, k = e - j * b;
    double acc = 0.0;
    for (int q = 0; q < b; ++q) {
      const double gq = a.base ? (double)a.base[q * b + k] : ((__popc(q & k) & 1) ? -hs : hs);
      acc = fma(m[j * P + b + q], gq, acc);
    }
    out[e] = (float)acc;
  }
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}

// 3 <= b <= MAXB <= 32: lane c < 2 MAXB keeps column c of [I - A | I + A] in
// registers, the system padded to MAXB with A = 0 beyond b (then Q is Q(b)
// bordered by the identity, and its leading b x b block is the same).  Each
// pivot broadcasts column i from lane i with readlane; no LDS, no barrier
// until Q is staged for the product.
template <int MAXB>
__device__ __forceinline__ void harp_reg_block(const HarpArgs& a, int64_t g, double* q_lds) {
  const int b = a.b, lane = threadIdx.x;
  const int8_t* th = a.theta + g * a.np;
  const double sc = (double)a.scale;
  const int c = lane < MAXB ? lane : lane - MAXB;  // column within its half
  const double sgn = lane < MAXB ? -1.0 : 1.0;     // I - A or I + A
  double col[MAXB];
#pragma unroll
  for (int r = 0; r < MAXB; ++r) {
    double arc = 0.0;
    if (r < b && c < b && lane < 2 * MAXB) {
      if (r < c) arc = sc * (double)th[harp_pidx(b, r, c)];
      else if (r > c) arc = -sc * (double)th[harp_pidx(b, c, r)];
    }
    col[r] = (r == c ? 1.0 : 0.0) + sgn * arc;
  }
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const double inv = 1.0 / readlane_f64(col[i], i);
    const double mine = col[i] * inv;
#pragma unroll
    for (int r = 0; r < MAXB; ++r)
      if (r != i) col[r] = fma(-readlane_f64(col[r], i), mine, col[r]);
    col[i] = mine;
  }
  // lanes MAXB .. 2 MAXB - 1 hold the columns of Q
  if (lane >= MAXB && lane < 2 * MAXB) {
#pragma unroll
    for (int r = 0; r < MAXB; ++r) q_lds[r * (MAXB + 1) + c] = col[r];
  }
  __syncthreads();
  const double hs = 1.0 / sqrt((double)b);
  float* out = a.out + g * b * b;
  if (!a.base && b == MAXB && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0) {
    // Sylvester G = H_b / sqrt(b) (b a power of two, so b is MAXB): row j of
    // Q G is the Walsh-Hadamard transform of row j of Q, b log2 b additions
    // in registers instead of b^2 products; lane j takes row j and stores it
    // as float4s (b^2 floats per block keep every row 16-byte aligned)
    if (lane < MAXB) {
      double r[MAXB];
#pragma unroll
      for (int q = 0; q < MAXB; ++q) r[q] = q_lds[lane * (MAXB + 1) + q];
#pragma unroll
      for (int h = 1; h < MAXB; h <<= 1)
#pragma unroll
        for (int i = 0; i < MAXB; ++i)
          if ((i & h) == 0) {
            const double x = r[i], y = r[i + h];
            r[i] = x + y;
            r[i + h] = x - y;
          }
      float4* o4 = reinterpret_cast<float4*>(out + lane * MAXB);
#pragma unroll
      for (int k = 0; k < MAXB / 4; ++k)
        o4[k] = make_float4((float)(r[4 * k] * hs), (float)(r[4 * k + 1] * hs), (float)(r[4 * k + 2] * hs),
                            (float)(r[4 * k + 3] * hs));
    }
    return;
  }
  for (int e = lane; e < b * b; e += kHpThreads) {
    const int j = e / b, k = e - j * b;
    double acc = 0.0;
    for (int q = 0; q < b; ++q) {
      const double gq = a.base ? (double)a.base[q * b + k] : ((__popc(q & k) & 1) ? -hs : hs);
      acc = fma(q_lds[j * (MAXB + 1) + q], gq, acc);
    }
    out[e] = (float)acc;
  }
}

template <int MAXB>
__global__ __launch_bounds__(kHpThreads) void harp_reg_kernel(HarpArgs a) {
  __shared__ double q_lds[MAXB * (MAXB + 1)];
  harp_reg_block<MAXB>(a, blockIdx.x, q_lds);
}

__global__ __launch_bounds__(kHpThreads) void harp_batch_kernel(HarpBatch bt) {
  __shared__ double q_lds[32 * 33];
  const int64_t w = blockIdx.x;
  int j = 0;
  while (j + 1 < bt.n && w >= bt.first[j + 1]) ++j;  // uniform over the workgroup
  const HarpArgs& a = bt.job[j];
  const int64_t g = w - bt.first[j];
  if (a.b <= 4) harp_reg_block<4>(a, g, q_lds);
  else if (a.b <= 8) harp_reg_block<8>(a, g, q_lds);
  else if (a.b <= 16) harp_reg_block<16>(a, g, q_lds);
  else harp_reg_block<32>(a, g, q_lds);
}

}  // namespace

hipError_t launch_harp_batch(const HarpBatch& a, hipStream_t s) {
  if (a.n < 1 || a.n > kHpMaxJobs || a.first[a.n] == 0) return a.n == 0 ? hipSuccess : hipErrorInvalidValue;
  hipLaunchKernelGGL(harp_batch_kernel, dim3((unsigned)a.first[a.n]), dim3(kHpThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_harp(const HarpArgs& a, hipStream_t s) {
  if (a.ngroups == 0) return hipSuccess;
  const dim3 grid((unsigned)a.ngroups), block(kHpThreads);
  if (a.b >= 3 && a.b <= 4) hipLaunchKernelGGL(harp_reg_kernel<4>, grid, block, 0, s, a);
  else if (a.b >= 5 && a.b <= 8) hipLaunchKernelGGL(harp_reg_kernel<8>, grid, block, 0, s, a);
  else if (a.b >= 9 && a.b <= 16) hipLaunchKernelGGL(harp_reg_kernel<16>, grid, block, 0, s, a);
  else if (a.b >= 17 && a.b <= 32) hipLaunchKernelGGL(harp_reg_kernel<32>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(harp_kernel, grid, block, harp_lds_bytes(a.b), s, a);
  return hipGetLastError();
}

}  // namespace brq
