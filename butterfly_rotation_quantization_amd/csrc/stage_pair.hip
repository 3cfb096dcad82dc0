// Two consecutive right-side stages in one launch, for few rows (stage.h).
#include "stage.h"

namespace brq {
namespace {

__device__ __forceinline__ float p2_load(const void* p, int t, int64_t i) {
  if (t == BRQ_F32) return static_cast<const float*>(p)[i];
  if (t == BRQ_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  return (float)static_cast<const _Float16*>(p)[i];
}

__device__ __forceinline__ void p2_store(void* p, int t, int64_t i, float v) {
  if (t == BRQ_F32) static_cast<float*>(p)[i] = v;
  else if (t == BRQ_BF16) static_cast<__bf16*>(p)[i] = (__bf16)v;  // nearest, ties to even
  else static_cast<_Float16*>(p)[i] = (_Float16)v;
}

// BO, BI: register bounds of the two radices (8 or 16).
template <int BO, int BI>
__global__ __launch_bounds__(256) void stage_pair2_kernel(P2Args a) {
  __shared__ float buf[256 * kP2Lines];  // per set: [line][outer index][inner index]
  const int n = a.bo * a.bi;
  const int u = threadIdx.x;
  const int sl = u / n, e = u - sl * n;
  int64_t sbk, lb;
  p2_tile(a, blockIdx.x, sbk, lb);
  const int64_t l0 = lb * kP2Lines;
  const int64_t s = sbk * a.sets + sl;
  const bool act = sl < a.sets && s < a.nsets;
  const int nl = (int)(a.lines - l0 < kP2Lines ? a.lines - l0 : kP2Lines);
  int64_t c = 0, hi = 0, lo = 0;
  if (act) p2_set(a, s, c, hi, lo);
  float* sb = buf + sl * (kP2Lines * n);
  // thread e: element (ea, eb) for the loads and stores; output oj of outer
  // group og (inner index og); output ij of inner group ig (outer index ig)
  const int ea = e / a.bi, eb = e - ea * a.bi;
  const int og = e / a.bo, oj = e - og * a.bo;
  const int ig = ea, ij = eb;
  int64_t pos = 0;
  float wo[BO], wi[BI], v[kP2Lines];
  float sg_out = 1.f;
#pragma unroll
  for (int k = 0; k < BO; ++k) wo[k] = 0.f;
#pragma unroll
  for (int k = 0; k < BI; ++k) wi[k] = 0.f;
  if (act) {
    pos = p2_pos(a, c, hi, lo, ea, eb);
#pragma unroll
    for (int l = 0; l < kP2Lines; ++l)
      if (l < nl) v[l] = p2_load(a.src, a.src_t, (l0 + l) * a.ld_src + pos);
    const float* ro = a.blk_o + p2_row_o(a, hi, lo, og, oj);
    const float* ri = a.blk_i + p2_row_i(a, hi, lo, ig, ij);
#pragma unroll
    for (int k = 0; k < BO; ++k)
      if (k < a.bo) wo[k] = ro[k];
    if (a.vec_i) {
#pragma unroll
      for (int k4 = 0; k4 < BI / 4; ++k4)
        if (4 * k4 < a.bi) {
          const float4 q = *reinterpret_cast<const float4*>(ri + 4 * k4);
          wi[4 * k4] = q.x;
          wi[4 * k4 + 1] = q.y;
          wi[4 * k4 + 2] = q.z;
          wi[4 * k4 + 3] = q.w;
        }
    } else {
#pragma unroll
      for (int k = 0; k < BI; ++k)
        if (k < a.bi) wi[k] = ri[k];
    }
    const float sg = a.sign_in ? a.sign_in[(uint32_t)(pos % a.d)] : 1.f;
    if (a.sign_out) sg_out = a.sign_out[(uint32_t)(pos % a.d)];  // loaded with the inputs
#pragma unroll
    for (int l = 0; l < kP2Lines; ++l)
      if (l < nl) sb[l * n + ea * a.bi + eb] = sg * v[l];
  }
  __syncthreads();
  for (int ph = 0; ph < 2; ++ph) {
    const bool outer = (ph == 0) != (a.inner_first != 0);
    float acc[kP2Lines];
    if (act) {
#pragma unroll
      for (int l = 0; l < kP2Lines; ++l) {
        if (l < nl) {
          float y = 0.f;
          if (outer) {
#pragma unroll
            for (int k = 0; k < BO; ++k)
              if (k < a.bo) y = fmaf(wo[k], sb[l * n + k * a.bi + og], y);
          } else {
#pragma unroll
            for (int k = 0; k < BI; ++k)
              if (k < a.bi) y = fmaf(wi[k], sb[l * n + ig * a.bi + k], y);
          }
          acc[l] = y;
        }
      }
    }
    __syncthreads();  // every input of the phase read
    if (act) {
      const int slot = outer ? oj * a.bi + og : ig * a.bi + ij;
#pragma unroll
      for (int l = 0; l < kP2Lines; ++l)
        if (l < nl) sb[l * n + slot] = acc[l];
    }
    __syncthreads();
  }
  if (act) {
#pragma unroll
    for (int l = 0; l < kP2Lines; ++l)
      if (l < nl) p2_store(a.dst, a.dst_t, (l0 + l) * a.ld_dst + pos, sg_out * sb[l * n + ea * a.bi + eb]);
  }
}

}  // namespace

hipError_t launch_stage_pair2(const P2Args& a, hipStream_t s) {
  const dim3 grid((unsigned)p2_blocks(a));
  if (a.bo <= 8 && a.bi <= 8) hipLaunchKernelGGL((stage_pair2_kernel<8, 8>), grid, dim3(256), 0, s, a);
  else if (a.bo <= 8) hipLaunchKernelGGL((stage_pair2_kernel<8, 16>), grid, dim3(256), 0, s, a);
  else if (a.bi <= 8) hipLaunchKernelGGL((stage_pair2_kernel<16, 8>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((stage_pair2_kernel<16, 16>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace brq
