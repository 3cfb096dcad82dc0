// Quantized linear layer kernels (qlinear.h).
#include "qlinear.h"

namespace brq {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));

// The 8 codes of inputs k .. k + 7 of one row (k a multiple of 8: they
// start on a byte and take BITS bytes).
template <int BITS>
__device__ __forceinline__ uint64_t ql_codes8(const uint8_t* p) {
  if constexpr (BITS == 2) return *reinterpret_cast<const uint16_t*>(p);
  if constexpr (BITS == 4) return *reinterpret_cast<const uint32_t*>(p);
  uint64_t v = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

template <int BITS, bool BF>
__global__ __launch_bounds__(kQlThreads) void qlinear_kernel(QlArgs a) {
  using V8 = typename std::conditional<BF, b8v, h8v>::type;
  constexpr int L = (1 << BITS) - 1;
  const QlTile t = ql_tile(a, blockIdx.x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t o = t.ct * kQlOut + 16 * w + lr;  // this lane's weight row (B operand)
  const int64_t tok = t.tt * kQlTok + lr;         // this lane's token (A operand)
  const bool tok_ok = tok < a.T;
  const int64_t k_beg = t.split * a.kc;
  const int64_t k_end = k_beg + a.kc < a.n ? k_beg + a.kc : a.n;
  const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + (tok_ok ? tok : 0) * a.ldx;
  const uint8_t* crow = a.codes + o * a.codes_ld;
  const float* srow = a.scales + o * a.scales_ld;
  const float invL = 1.0f / (float)L;
  f4v acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t g0 = k_beg; g0 < k_end; g0 += a.group) {
    f4v d = {0.f, 0.f, 0.f, 0.f};
    for (int64_t k = g0 + 8 * lg; k < g0 + a.group; k += 32) {
      V8 av;
      if (tok_ok) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xrow + k);
        av = __builtin_bit_cast(V8, raw);
      } else {
        av = __builtin_bit_cast(V8, make_uint4(0u, 0u, 0u, 0u));
      }
      const uint64_t c8 = ql_codes8<BITS>(crow + k * BITS / 8);
      V8 bv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 2 * (int)((c8 >> (BITS * i)) & L) - L;
        if constexpr (BF) bv[i] = (__bf16)(float)q;
        else bv[i] = (_Float16)q;
      }
      if constexpr (BF) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, d, 0, 0, 0);
      else d = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, d, 0, 0, 0);
    }
    // D reg i: token 4 lg + i, output lr: scale alpha(o, group) / L
    const float s = srow[g0 / a.group] * invL;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(d[i], s, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tk = t.tt * kQlTok + 4 * lg + i;
    if (tk < a.T) a.part[((int64_t)t.split * a.T + tk) * a.m + o] = acc[i];
  }
}

__global__ void ql_reduce_kernel(const float* part, int splits, int64_t T, int64_t m, void* out,
                                 int ot, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * m) return;
  const int64_t t = i / m, o = i - t * m;
  float s = 0.f;
  for (int p = 0; p < splits; ++p) s += part[(int64_t)p * T * m + i];
  const int64_t j = t * ldo + o;
  if (ot == BRQ_F32) {
    static_cast<float*>(out)[j] = s;
  } else if (ot == BRQ_F16) {
    static_cast<_Float16*>(out)[j] = (_Float16)s;
  } else {
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) > 0x7f800000u) u |= 0x400000u;  // keep NaN a quiet NaN
    else u += 0x7fffu + ((u >> 16) & 1u);                   // nearest, ties to even
    static_cast<uint16_t*>(out)[j] = (uint16_t)(u >> 16);
  }
}

template <int BITS>
hipError_t launch_b(const QlArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)ql_blocks(a));
  if (a.xt == BRQ_BF16) hipLaunchKernelGGL((qlinear_kernel<BITS, true>), grid, dim3(kQlThreads), 0, s, a);
  else hipLaunchKernelGGL((qlinear_kernel<BITS, false>), grid, dim3(kQlThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qlinear(const QlArgs& a, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_b<2>(a, s);
    case 3: return launch_b<3>(a, s);
    case 4: return launch_b<4>(a, s);
    case 5: return launch_b<5>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ql_reduce(const float* part, int splits, int64_t T, int64_t m, void* out, int ot,
                            int64_t ldo, hipStream_t s) {
  const int64_t n = T * m;
  hipLaunchKernelGGL(ql_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                     splits, T, m, out, ot, ldo);
  return hipGetLastError();
}

}  // namespace brq
