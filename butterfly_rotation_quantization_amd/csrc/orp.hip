// ORP GEO quantizer kernels ([ORPQuant] technical summary, section 2; the
// layout and shared index helpers are in orp.h).
//
// Quantize, per group of g inputs of a row (w_p = w * s, s the optional
// per-input-channel smoothing vector, one float32 product):
//   alpha = max |w_p|; u = w_p * fl(1 / alpha) in float32;
//   b1 = the level of the asymmetric power-of-two lattice with zero nearest
//        to u (2^(b-1) negative levels -1 .. -2^-(2^(b-1)-1), zero, 2^(b-1)-1
//        positive ones 1 .. 2^-(2^(b-1)-2); codes index them in ascending
//        order; a tie goes to the lower code);
//   pairs (i, i + S) inside micro-blocks of 2S: d = w_p[i+S] b1[i] - w_p[i] b1[i+S]
//        (the residual's component along (-b1[i+S], b1[i])), sigma = +1 if
//        d >= 0 else -1, b2 = sigma * (-b1[i+S], b1[i]);
//   c1 = <w_p, b1> / ||b1||^2, c2 = <w_p, b2> / ||b1||^2 = sum |d| / ||b1||^2
//        (||b2|| = ||b1||; both 0 for a zero group).
// Dequantize: w_p^ = c1 b1 + c2 b2, one rounding (the product c1 b1 is exact).
//
// The level decision works on the bits of u: |u| = m 2^E with m in [1, 2)
// is nearest to 2^(E+1) when m > 1.5 (m = 1.5 is a tie: up on the negative
// side, whose lower code is the larger magnitude); below the smallest
// magnitude 2^-k the choice is between it and zero at the midpoint
// 2^-(k+1).  Products of float32 values with powers of two are exact, so
// the sign of d is exact.
#include "orp.h"

namespace brq {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef float f4 __attribute__((ext_vector_type(4)));

// Eight consecutive elements (16-byte aligned) as float.
__device__ __forceinline__ void load8(const void* base, int t, int64_t off, float (&v)[8]) {
  if (t == BRQ_F32) {
    const f4* p = reinterpret_cast<const f4*>(static_cast<const float*>(base) + off);
    const f4 x0 = p[0], x1 = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = x0[e];
      v[4 + e] = x1[e];
    }
    return;
  }
  const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = t == BRQ_BF16 ? bf16_lo(w[e]) : f16_lo(w[e]);
    v[2 * e + 1] = t == BRQ_BF16 ? bf16_hi(w[e]) : f16_hi(w[e]);
  }
}

__device__ __forceinline__ uint32_t to_bf16(float f) {  // nearest, ties to even
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ void store8(void* base, int t, int64_t off, const float (&v)[8]) {
  if (t == BRQ_F32) {
    f4* p = reinterpret_cast<f4*>(static_cast<float*>(base) + off);
    p[0] = f4{v[0], v[1], v[2], v[3]};
    p[1] = f4{v[4], v[5], v[6], v[7]};
    return;
  }
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = t == BRQ_BF16 ? (to_bf16(v[2 * e]) | (to_bf16(v[2 * e + 1]) << 16))
                         : (to_f16(v[2 * e]) | (to_f16(v[2 * e + 1]) << 16));
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Reduction over the lpg lanes of a group (lpg a power of two, groups aligned
// to lpg lanes); every lane of the group ends with the result.
template <bool MAX>
__device__ __forceinline__ float group_reduce(float x, int lpg) {
  for (int off = 1; off < lpg; off <<= 1) {
    const float y = __shfl_xor(x, off);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  return x;
}

// Lattice level of u: its code and its value.
template <int BITS>
__device__ __forceinline__ uint32_t level_of(float u, float* val) {
  constexpr int H = 1 << (BITS - 1);
  const uint32_t ub = __float_as_uint(u);
  const uint32_t neg = ub >> 31;
  const uint32_t ab = ub & 0x7fffffffu;
  const int kmax = neg ? H - 1 : H - 2;
  const uint32_t man = ab & 0x7fffffu;
  const int e = (int)(ab >> 23) - 127;
  const int up = (man > 0x400000u) | ((man == 0x400000u) & neg);
  int k = -(e + up);
  k = k < 0 ? 0 : k;
  bool zero = false;
  if (k > kmax) {
    // between 2^-kmax and zero: the midpoint is 2^-(kmax+1); a tie goes to
    // the lower code (zero on the positive side, -2^-kmax on the negative)
    const uint32_t mid = (uint32_t)(127 - kmax - 1) << 23;
    zero = ab < mid || (ab == mid && !neg);
    k = kmax;
  }
  if (zero) {
    *val = 0.0f;
    return (uint32_t)H;
  }
  *val = __uint_as_float((neg << 31) | ((uint32_t)(127 - k) << 23));
  return neg ? (uint32_t)k : (uint32_t)((1 << BITS) - 1 - k);
}

template <int BITS>
__device__ __forceinline__ float level_value(uint32_t code) {
  constexpr int H = 1 << (BITS - 1);
  if (code == (uint32_t)H) return 0.0f;
  const bool neg = code < (uint32_t)H;
  const int k = neg ? (int)code : (1 << BITS) - 1 - (int)code;
  return __uint_as_float(((uint32_t)neg << 31) | ((uint32_t)(127 - k) << 23));
}

// Store `BITS` bytes holding eight BITS-bit codes, LSB first.
template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, uint64_t packed) {
  if (BITS == 2) {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)packed;
  } else if (BITS == 4) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)packed;
  } else {
#pragma unroll
    for (int b = 0; b < BITS; ++b) p[b] = (uint8_t)(packed >> (8 * b));
  }
}

template <int BITS>
__device__ __forceinline__ uint64_t load_codes(const uint8_t* p) {
  if (BITS == 2) return *reinterpret_cast<const uint16_t*>(p);
  if (BITS == 4) return *reinterpret_cast<const uint32_t*>(p);
  uint64_t x = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) x |= (uint64_t)p[b] << (8 * b);
  return x;
}

// SIN: the pair stride when the micro-block lies inside a lane's eight
// elements (1, 2 or 4); 0 when pairs span lanes (stride >= 8).
template <int BITS, int SIN>
__global__ __launch_bounds__(kOrpThreads) void orp_quant_kernel(OrpArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kOrpThreads / 64) + (threadIdx.x >> 6);
  if (wave >= a.m * a.chunks) return;  // uniform over the wavefront
  int64_t row, c0;
  orp_wave(a, wave, &row, &c0);
  const int64_t col = c0 + kOrpPerLane * lane;
  const bool valid = col < a.n;  // n is a multiple of the group, chunks of whole groups
  const int lpg = a.group / kOrpPerLane;
  float v[8];
  if (valid) {
    load8(a.w, a.wt, row * a.ldw + col, v);
    if (a.smooth) {
      const f4* sp = reinterpret_cast<const f4*>(a.smooth + col);
      const f4 s0 = sp[0], s1 = sp[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] *= s0[e];
        v[4 + e] *= s1[e];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
  am = group_reduce<true>(am, lpg);
  const float k = am > 0.0f ? 1.0f / am : 0.0f;
  float b1[8];
  uint64_t packed = 0;
  float dot = 0.0f, nn = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t c = level_of<BITS>(v[j] * k, &b1[j]);
    packed |= (uint64_t)c << (BITS * j);
    dot = fmaf(v[j], b1[j], dot);
    nn = fmaf(b1[j], b1[j], nn);
  }
  // pair signs and sum |d| (each pair counted once)
  float sabs = 0.0f;
  uint32_t sbits = 0;
  bool first_half = true;
  if (SIN > 0) {
#pragma unroll
    for (int q = 0; q < 8 / (2 * SIN); ++q)
#pragma unroll
      for (int r = 0; r < SIN; ++r) {
        const int i = q * 2 * SIN + r, i2 = i + SIN;
        const float d = v[i2] * b1[i] - v[i] * b1[i2];
        sabs += fabsf(d);
        sbits |= (d < 0.0f ? 1u : 0u) << (q * SIN + r);
      }
  } else {
    const int xm = a.stride / kOrpPerLane;
    first_half = ((lane & (lpg - 1)) & xm) == 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float vp = __shfl_xor(v[j], xm);
      const float bp = __shfl_xor(b1[j], xm);
      // first half: this lane holds entry i, the partner i + S
      const float d = vp * b1[j] - v[j] * bp;
      if (first_half) {
        sabs += fabsf(d);
        sbits |= (d < 0.0f ? 1u : 0u) << j;
      }
    }
  }
  dot = group_reduce<false>(dot, lpg);
  nn = group_reduce<false>(nn, lpg);
  sabs = group_reduce<false>(sabs, lpg);
  // the neighbour's nibble (in-lane pairs: four pair bits per lane)
  const uint32_t nb = SIN > 0 ? (uint32_t)__shfl_xor((int)sbits, 1) : 0u;
  if (!valid) return;
  store_codes<BITS>(a.codes + row * (a.n * BITS / 8) + col * BITS / 8, packed);
  uint8_t* srow = a.signs + row * (a.n / 16);
  if (SIN > 0) {
    if ((lane & 1) == 0) srow[col / 16] = (uint8_t)(sbits | (nb << 4));
  } else if (first_half) {
    srow[orp_pair(col, a.stride) / 8] = (uint8_t)sbits;
  }
  if ((lane & (lpg - 1)) == 0) {
    const float c1 = nn > 0.0f ? dot / nn : 0.0f;
    const float c2 = nn > 0.0f ? sabs / nn : 0.0f;
    *reinterpret_cast<float2*>(a.coef + 2 * (row * (a.n / a.group) + col / a.group)) =
        make_float2(c1, c2);
  }
}

template <int BITS, int SIN>
__global__ __launch_bounds__(kOrpThreads) void orp_dequant_kernel(OrpArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kOrpThreads / 64) + (threadIdx.x >> 6);
  if (wave >= a.m * a.chunks) return;  // uniform over the wavefront
  int64_t row, c0;
  orp_wave(a, wave, &row, &c0);
  const int64_t col = c0 + kOrpPerLane * lane;
  const bool valid = col < a.n;
  const int lpg = a.group / kOrpPerLane;
  float b1[8];
  uint64_t packed = 0;
  const uint8_t* srow = a.signs + row * (a.n / 16);
  if (valid) packed = load_codes<BITS>(a.codes + row * (a.n * BITS / 8) + col * BITS / 8);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    b1[j] = level_value<BITS>((uint32_t)(packed >> (BITS * j)) & ((1u << BITS) - 1));
  float b2[8];
  if (SIN > 0) {
    const uint32_t sb = valid ? (uint32_t)(srow[col / 16] >> (4 * (lane & 1))) : 0u;
#pragma unroll
    for (int q = 0; q < 8 / (2 * SIN); ++q)
#pragma unroll
      for (int r = 0; r < SIN; ++r) {
        const int i = q * 2 * SIN + r, i2 = i + SIN;
        const float sg = ((sb >> (q * SIN + r)) & 1u) ? -1.0f : 1.0f;
        b2[i] = -sg * b1[i2];
        b2[i2] = sg * b1[i];
      }
  } else {
    const int xm = a.stride / kOrpPerLane;
    const bool first_half = ((lane & (lpg - 1)) & xm) == 0;
    // the pair's sign byte sits at the pair number of its first entry
    const int64_t first_col = first_half ? col : col - a.stride;
    const uint32_t sb = valid ? (uint32_t)srow[orp_pair(first_col, a.stride) / 8] : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float bp = __shfl_xor(b1[j], xm);
      const float sg = ((sb >> j) & 1u) ? -1.0f : 1.0f;
      b2[j] = first_half ? -sg * bp : sg * bp;
    }
  }
  if (!valid) return;
  const float2 c = *reinterpret_cast<const float2*>(a.coef + 2 * (row * (a.n / a.group) + col / a.group));
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = fmaf(c.y, b2[j], c.x * b1[j]);
  store8(a.out, a.ot, row * a.ldo + col, o);
}

template <int BITS, int SIN>
hipError_t launch_bs(const OrpArgs& a, bool quant, hipStream_t s) {
  const dim3 grid((unsigned)orp_blocks(a)), block(kOrpThreads);
  if (quant)
    hipLaunchKernelGGL((orp_quant_kernel<BITS, SIN>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((orp_dequant_kernel<BITS, SIN>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_b(const OrpArgs& a, bool quant, hipStream_t s) {
  switch (a.stride) {
    case 1: return launch_bs<BITS, 1>(a, quant, s);
    case 2: return launch_bs<BITS, 2>(a, quant, s);
    case 4: return launch_bs<BITS, 4>(a, quant, s);
    default: return launch_bs<BITS, 0>(a, quant, s);
  }
}

hipError_t launch_any(const OrpArgs& a, bool quant, hipStream_t s) {
  if (orp_waves(a) == 0) return hipSuccess;
  switch (a.bits) {
    case 2: return launch_b<2>(a, quant, s);
    case 3: return launch_b<3>(a, quant, s);
    case 4: return launch_b<4>(a, quant, s);
    case 5: return launch_b<5>(a, quant, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_orp_quant(const OrpArgs& a, hipStream_t s) { return launch_any(a, true, s); }
hipError_t launch_orp_dequant(const OrpArgs& a, hipStream_t s) { return launch_any(a, false, s); }

}  // namespace brq
