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

// Eight consecutive elements (16-byte aligned): the raw bytes (two 16-byte
// pieces for float32, one for 16-bit types), then as float.
template <int WT>
__device__ __forceinline__ void load_raw(const void* base, int64_t off, uint4 (&r)[2]) {
  if (WT == BRQ_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
    r[0] = p[0];
    r[1] = p[1];
  } else {
    r[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    r[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int WT>
__device__ __forceinline__ void unpack_raw(const uint4 (&r)[2], float (&v)[8]) {
  if (WT == BRQ_F32) {
    const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(w[e]);
    return;
  }
  const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = WT == BRQ_BF16 ? bf16_lo(w[e]) : f16_lo(w[e]);
    v[2 * e + 1] = WT == BRQ_BF16 ? bf16_hi(w[e]) : f16_hi(w[e]);
  }
}

__device__ __forceinline__ uint32_t to_bf16(float f) {  // nearest, ties to even
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int OT>
__device__ __forceinline__ void store8(void* base, int64_t off, const float (&v)[8]) {
  if (OT == BRQ_F32) {
    f4* p = reinterpret_cast<f4*>(static_cast<float*>(base) + off);
    p[0] = f4{v[0], v[1], v[2], v[3]};
    p[1] = f4{v[4], v[5], v[6], v[7]};
    return;
  }
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = OT == BRQ_BF16 ? (to_bf16(v[2 * e]) | (to_bf16(v[2 * e + 1]) << 16))
                          : (to_f16(v[2 * e]) | (to_f16(v[2 * e + 1]) << 16));
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Reduction over the lpg lanes of a group (lpg a power of two, groups aligned
// to lpg lanes); every lane of the group ends with the result.  Within a row
// of 16 lanes the steps are DPP moves (swap neighbours, swap pairs, mirror
// each half row, mirror the row), beyond it shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <bool MAX>
__device__ __forceinline__ float group_reduce(float x, int lpg) {
  auto op = [](float p, float q) { return MAX ? fmaxf(p, q) : p + q; };
  if (lpg > 1) x = op(x, dpp<0xb1>(x));   // quad_perm [1,0,3,2]
  if (lpg > 2) x = op(x, dpp<0x4e>(x));   // quad_perm [2,3,0,1]
  if (lpg > 4) x = op(x, dpp<0x141>(x));  // row_half_mirror
  if (lpg > 8) x = op(x, dpp<0x140>(x));  // row_mirror
  if (lpg > 16) x = op(x, __shfl_xor(x, 16));
  if (lpg > 32) x = op(x, __shfl_xor(x, 32));
  return x;
}

// Lattice level of u: its code and its value, without branches.  With
// |u| = m 2^E, adding 0x3fffff (+1 on the negative side) to the bits of |u|
// carries into the exponent exactly when m > 1.5 (m >= 1.5 on the negative
// side, where the lower code is the larger magnitude), which rounds |u| to
// its nearest power of two 2^-k.  Below the smallest magnitude 2^-kmax the
// choice is zero or 2^-kmax at the midpoint 2^-(kmax+1), a tie again going
// to the lower code (zero on the positive side).
template <int BITS>
__device__ __forceinline__ uint32_t level_of(float u, float* val) {
  constexpr int H = 1 << (BITS - 1);
  const uint32_t ub = __float_as_uint(u);
  const uint32_t neg = ub >> 31;
  const uint32_t ab = ub & 0x7fffffffu;
  const int kmax = H - 2 + (int)neg;
  int k = 127 - (int)((ab + 0x3fffffu + neg) >> 23);
  k = k < 0 ? 0 : (k > kmax ? kmax : k);
  const uint32_t mid = (uint32_t)(126 - kmax) << 23;
  const bool zero = ab + neg <= mid;
  const uint32_t bits = (neg << 31) | ((uint32_t)(127 - k) << 23);
  *val = zero ? 0.0f : __uint_as_float(bits);
  const uint32_t code = neg ? (uint32_t)k : (uint32_t)((1 << BITS) - 1 - k);
  return zero ? (uint32_t)H : code;
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

// One chunk of a row: the quantizer on a lane's eight preconditioned values
// v (zeros for a lane past the row's end, which stores nothing).
// SIN: the pair stride when the micro-block lies inside a lane's eight
// elements (1, 2 or 4); 0 when pairs span lanes (stride >= 8).
template <int BITS, int SIN>
__device__ __forceinline__ void quant_chunk(const OrpArgs& a, int lane, int64_t row, uint32_t col,
                                            bool valid, const float (&v)[8]) {
  const int lpg = a.group / kOrpPerLane;
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
  store_codes<BITS>(a.codes + row * a.codes_ld + col * BITS / 8, packed);
  uint8_t* srow = a.signs + row * a.signs_ld;
  if (SIN > 0) {
    if ((lane & 1) == 0) srow[col >> 4] = (uint8_t)(sbits | (nb << 4));
  } else if (first_half) {
    srow[orp_pair_lg(col, a.lg_stride) >> 3] = (uint8_t)sbits;
  }
  if ((lane & (lpg - 1)) == 0) {
    const float c1 = nn > 0.0f ? dot / nn : 0.0f;
    const float c2 = nn > 0.0f ? sabs / nn : 0.0f;
    *reinterpret_cast<float2*>(a.coef + row * a.coef_ld + 2 * (col >> a.lg_group)) =
        make_float2(c1, c2);
  }
}

template <int BITS, int SIN, int WT>
__global__ __launch_bounds__(kOrpThreads) void orp_quant_kernel(OrpArgs a) {
  constexpr int C = kOrpChunksPerWave;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kOrpThreads / 64) + (threadIdx.x >> 6);
  const int64_t total = orp_total_chunks(a);
  const int64_t ci0 = wave * C;
  if (ci0 >= total) return;  // uniform over the wavefront
  uint4 raw[C][2];
  f4 sm[C][2];
  // the chunks' rows and first columns: one division per wavefront, then steps
  int64_t rows[C];
  uint32_t c0s[C];
  {
    int64_t row, c0;
    orp_chunk(a, ci0, &row, &c0);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      rows[j] = row;
      c0s[j] = (uint32_t)c0;
      c0 += kOrpChunk;
      if (c0 >= a.n) {
        c0 = 0;
        ++row;
      }
    }
  }
  const uint32_t n32 = (uint32_t)a.n;
  // every chunk's loads in flight before the first is used
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const uint32_t col = c0s[j] + kOrpPerLane * lane;
    if (ci0 + j < total && col < n32) {
      load_raw<WT>(a.w, rows[j] * a.ldw + col, raw[j]);
      if (a.smooth) {
        const f4* sp = reinterpret_cast<const f4*>(a.smooth + col);
        sm[j][0] = sp[0];
        sm[j][1] = sp[1];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    if (ci0 + j >= total) break;  // uniform
    const int64_t row = rows[j];
    const uint32_t col = c0s[j] + kOrpPerLane * lane;
    const bool valid = col < n32;  // n is a multiple of the group, chunks of whole groups
    float v[8];
    if (valid) {
      unpack_raw<WT>(raw[j], v);
      if (a.smooth) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] *= sm[j][0][e];
          v[4 + e] *= sm[j][1][e];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    quant_chunk<BITS, SIN>(a, lane, row, col, valid, v);
  }
}

template <int BITS, int SIN, int OT>
__global__ __launch_bounds__(kOrpThreads) void orp_dequant_kernel(OrpArgs a) {
  constexpr int C = kOrpChunksPerWave;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kOrpThreads / 64) + (threadIdx.x >> 6);
  const int64_t total = orp_total_chunks(a);
  const int64_t ci0 = wave * C;
  if (ci0 >= total) return;  // uniform over the wavefront
  const int lpg = a.group / kOrpPerLane;
  const int xm = SIN > 0 ? 0 : a.stride / kOrpPerLane;
  const bool first_half = SIN > 0 || ((lane & (lpg - 1)) & xm) == 0;
  uint64_t packed[C];
  uint32_t sb[C];
  float2 cf[C];
  int64_t rows[C];
  uint32_t c0s[C];
  {
    int64_t row, c0;
    orp_chunk(a, ci0, &row, &c0);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      rows[j] = row;
      c0s[j] = (uint32_t)c0;
      c0 += kOrpChunk;
      if (c0 >= a.n) {
        c0 = 0;
        ++row;
      }
    }
  }
  const uint32_t n32 = (uint32_t)a.n;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    packed[j] = 0;
    sb[j] = 0;
    cf[j] = make_float2(0.f, 0.f);
    const int64_t row = rows[j];
    const uint32_t col = c0s[j] + kOrpPerLane * lane;
    if (ci0 + j < total && col < n32) {
      packed[j] = load_codes<BITS>(a.codes + row * a.codes_ld + col * BITS / 8);
      const uint8_t* srow = a.signs + row * a.signs_ld;
      if (SIN > 0) {
        sb[j] = (uint32_t)(srow[col >> 4] >> (4 * (lane & 1)));
      } else {
        // the pair's sign byte sits at the pair number of its first entry
        const uint32_t first_col = first_half ? col : col - (uint32_t)a.stride;
        sb[j] = (uint32_t)srow[orp_pair_lg(first_col, a.lg_stride) >> 3];
      }
      cf[j] = *reinterpret_cast<const float2*>(a.coef + row * a.coef_ld + 2 * (col >> a.lg_group));
    }
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    if (ci0 + j >= total) break;  // uniform
    const int64_t row = rows[j];
    const uint32_t col = c0s[j] + kOrpPerLane * lane;
    float b1[8], b2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      b1[e] = level_value<BITS>((uint32_t)(packed[j] >> (BITS * e)) & ((1u << BITS) - 1));
    if (SIN > 0) {
#pragma unroll
      for (int q = 0; q < 8 / (2 * SIN); ++q)
#pragma unroll
        for (int r = 0; r < SIN; ++r) {
          const int i = q * 2 * SIN + r, i2 = i + SIN;
          const float sg = ((sb[j] >> (q * SIN + r)) & 1u) ? -1.0f : 1.0f;
          b2[i] = -sg * b1[i2];
          b2[i2] = sg * b1[i];
        }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bp = __shfl_xor(b1[e], xm);
        const float sg = ((sb[j] >> e) & 1u) ? -1.0f : 1.0f;
        b2[e] = first_half ? -sg * bp : sg * bp;
      }
    }
    if (col >= n32) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = fmaf(cf[j].y, b2[e], cf[j].x * b1[e]);
      // the float32 result is what a 16-bit output rounds (the compiler would
      // otherwise fold the multiply-add and the conversion into one rounding)
      asm volatile("" : "+v"(o[e]));
    }
    store8<OT>(a.out, row * a.ldo + col, o);
  }
}

template <int BITS, int SIN, int T>
hipError_t launch_bst(const OrpArgs& a, bool quant, hipStream_t s) {
  const dim3 grid((unsigned)orp_blocks(a)), block(kOrpThreads);
  if (quant)
    hipLaunchKernelGGL((orp_quant_kernel<BITS, SIN, T>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((orp_dequant_kernel<BITS, SIN, T>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BITS, int SIN>
hipError_t launch_bs(const OrpArgs& a, bool quant, hipStream_t s) {
  const int t = quant ? a.wt : a.ot;
  if (t == BRQ_F32) return launch_bst<BITS, SIN, BRQ_F32>(a, quant, s);
  if (t == BRQ_BF16) return launch_bst<BITS, SIN, BRQ_BF16>(a, quant, s);
  return launch_bst<BITS, SIN, BRQ_F16>(a, quant, s);
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
