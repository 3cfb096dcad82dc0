// Row Hadamard kernels (see rowhad.h for the data movement).
//
// Transform ([RHT] randomised Hadamard transform; [HARP] technical summary
// 2.1 with Sylvester blocks): each d-chunk x of a row becomes
// H_d D x / sqrt(d), with D the plan's signs and H_d[i][k] = (-1)^popcount(i&k).
// H_d is a product of radix-2 stages, one per index bit; the stage on bit p
// maps the pair (x[i], x[i + 2^p]) (bit p of i clear) to their sum and
// difference, and the stages commute.  The inverse is D H_d / sqrt(d).
//
// Quantizers ([HARP] and [PolarQuant] pages; the same formulas as the tile
// pass): absmax codes rint(v * h / alpha + h) clamped to [0, 2^b - 1] with
// h = (2^b - 1) / 2 and fp32 alpha = max |v| per group; the norm codebook maps
// z = v * sqrt(g) / r to the number of thresholds below it, r the group's
// 2-norm stored as fp16.
#include <utility>

#include "rowhad.h"

namespace brq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 hf2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// Two floats to two 16-bit values in one word (lo first), nearest, ties to
// even: one packed conversion.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v{lo, hi}), bf2v));
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v{lo, hi}), hf2v));
}

// 16 consecutive elements (16-byte aligned) as float.
__device__ __forceinline__ void load16(const void* base, int t, int64_t off, float (&v)[16]) {
  if (t == BRQ_F32) {
    const f4* p = reinterpret_cast<const f4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f4 x = p[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint4 x0 = p[0], x1 = p[1];  // both loads in flight before any conversion
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (t == BRQ_BF16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[2 * e] = bf16_lo(w[e]);
        v[2 * e + 1] = bf16_hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[2 * e] = f16_lo(w[e]);
        v[2 * e + 1] = f16_hi(w[e]);
      }
    }
  }
}

__device__ __forceinline__ void store16(void* base, int t, int64_t off, const float (&v)[16]) {
  if (t == BRQ_F32) {
    f4* p = reinterpret_cast<f4*>(static_cast<float*>(base) + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = f4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  } else {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = v[8 * q + 2 * e], hi = v[8 * q + 2 * e + 1];
        w[e] = t == BRQ_BF16 ? pack_bf16(lo, hi) : pack_f16(lo, hi);
      }
      p[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Radix-2 stages on register bits [q0, 4): butterflies between registers
// (q0 is a constant once the round loop is unrolled).
__device__ __forceinline__ void butterflies(float (&v)[16], int q0) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q >= q0)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!((j >> q) & 1)) {
        const float a = v[j], b = v[j | (1 << q)];
        v[j] = a + b;
        v[j | (1 << q)] = a - b;
      }
}

// Reduction over the lanes of one quantizer group (lpg consecutive lanes, a
// power of two, groups aligned to lpg).  Within a row of 16 lanes the steps
// are DPP moves: swap neighbours, swap pairs, then mirror each half row and
// the whole row, which pairs quads and then halves; wider groups use
// cross-row shuffles.  Every lane of a group ends with the same value (the
// same pairwise tree as xor steps 1, 2, 4, 8).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <bool MAX>
__device__ __forceinline__ float group_reduce(float x, int lpg) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if (lpg > 1) x = op(x, dpp<0xb1>(x));   // quad_perm [1,0,3,2]
  if (lpg > 2) x = op(x, dpp<0x4e>(x));   // quad_perm [2,3,0,1]
  if (lpg > 4) x = op(x, dpp<0x141>(x));  // row_half_mirror
  if (lpg > 8) x = op(x, dpp<0x140>(x));  // row_mirror
  if (lpg > 16) x = op(x, __shfl_xor(x, 16, 64));
  if (lpg > 32) x = op(x, __shfl_xor(x, 32, 64));
  return x;
}

// The 16 codes of one thread: 2 * BITS bytes at a 2 * BITS-aligned offset.
template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&c)[16]) {
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bit = j * BITS, wi = bit >> 5, sh = bit & 31;
    w[wi] |= c[j] << sh;
    if (sh + BITS > 32) w[wi + 1] |= c[j] >> (32 - sh);
  }
  if constexpr ((BITS & 1) == 0) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
    for (int k = 0; k < BITS / 2; ++k) q[k] = w[k];
  } else {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int k = 0; k < BITS; ++k) q[k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
  }
}

// The 16 codes of one thread as byte offsets into a float table (4 c): each
// is a shift and a mask of its word, or of the two words it straddles.
template <int BITS>
__device__ __forceinline__ void load_code_offsets(const uint8_t* p, uint32_t (&o)[16]) {
  uint32_t w[3] = {0u, 0u, 0u};
  if constexpr ((BITS & 1) == 0) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int k = 0; k < BITS / 2; ++k) w[k] = q[k];
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k >> 1] |= (uint32_t)q[k] << (16 * (k & 1));
  }
  constexpr uint32_t mask4 = ((1u << BITS) - 1u) << 2;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bit = j * BITS, wi = bit >> 5, sh = bit & 31;
    if (sh + BITS > 32) {
      o[j] = (((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) << 2) & mask4;
    } else if (sh >= 2) {
      o[j] = (w[wi] >> (sh - 2)) & mask4;
    } else {
      o[j] = (w[wi] << (2 - sh)) & mask4;
    }
  }
}

// BITS: the code width of the quantize and dequantize modes (0 for rotate);
// BITS2: the re-quantizer's code width (RH_REQUANT only).
template <int L2D, int MODE, int BITS, int BITS2>
__global__ __launch_bounds__(kRhThreads) void rowhad_kernel(RhArgs a) {
  __shared__ float lds[kRhLds];  // one buffer: more workgroups per CU beat a saved barrier
  // quantize: codebook bins {own threshold (or +inf), thresholds below};
  // dequantize: the level values (centroid / sqrt(g), or code / h - 1)
  constexpr bool DEQ = MODE == RH_DEQUANT || MODE == RH_REQUANT;  // codes in
  constexpr bool QOUT = MODE == RH_QUANT || MODE == RH_REQUANT;    // codes out
  __shared__ float2 tab[MODE == RH_QUANT ? kRhBins : 1];
  __shared__ float lev[DEQ ? kMaxLevels : 1];
  constexpr int R = rh_rounds(L2D);
  constexpr int LV = (1 << BITS) - 1;
  const RhPos p = rh_pos(a, blockIdx.x, threadIdx.x);
  const int lpg = (MODE == RH_REQUANT ? a.group2 : a.group) / 16;  // lanes per output group
  const bool bins = MODE == RH_QUANT && a.qkind == BRQ_CODEBOOK_NORM && a.bin_s != 0.f;
  // The global loads are issued first; the quantizer tables are built while
  // they are in flight.
  auto build_tables = [&]() {
    if (MODE == RH_QUANT && bins) tab[threadIdx.x] = a.bintab[threadIdx.x];  // built on the host
    if (DEQ && threadIdx.x <= LV) {  // the levels carry the transform's 1 / sqrt(d)
      const int c = threadIdx.x;
      lev[c] = (a.qkind == BRQ_ABSMAX ? (float)c / a.h - 1.0f : a.cent[c] / a.sqrt_g) * a.scale;
    }
  };
  float v[16];

  // ---- prologue: load or unpack + dequantize, then the signs (forward)
  // A dead thread (past the last chunk) reads valid memory, transforms it in
  // its own chunk's LDS area and stores nothing; its quantizer groups hold no
  // live lane.
  if (!DEQ) {
    load16(a.x, a.xt, p.row * a.ldx + p.col0, v);
    build_tables();
  } else {
    uint32_t c[16];  // byte offsets into lev
    load_code_offsets<BITS>(a.in_codes + p.row * a.codes_ld + p.col0 * BITS / 8, c);
    const int64_t sidx = p.row * a.scales_ld + p.col0 / a.group;
    const float scale = a.qkind == BRQ_ABSMAX ? static_cast<const float*>(a.in_scales)[sidx]
                                              : (float)static_cast<const _Float16*>(a.in_scales)[sidx];
    build_tables();
    __syncthreads();  // the level table
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = scale * *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(lev) + c[j]);
  }
  // The transform's 1 / sqrt(d): folded into the signs (rotate), into the
  // level table (dequantize), or left out (quantize: the codes depend only on
  // v / stat, and the stored statistic is scaled instead).
  if (!a.inverse && a.signs) {
    const float* sg = MODE == RH_ROTATE ? a.signs_s : a.signs;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= sg[16 * p.cu + j];
  }

  // ---- transform: per round, butterflies on its new bits, then an LDS
  // transpose to the next round's layout (the last one back to natural order)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!a.identity) butterflies(v, 4 - rh_nnew(L2D, r));
    if (R > 1) {
      const int rn = r + 1 < R ? r + 1 : 0;
      float* wb = lds + rh_lds_base(L2D, r, p.cw, p.cu);
      const float* rb = lds + rh_lds_base(L2D, rn, p.cw, p.cu);
#pragma unroll
      for (int j = 0; j < 16; ++j) wb[rh_lds_off(L2D, r, j)] = v[j];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = rb[rh_lds_off(L2D, rn, j)];
      if (r + 1 < R) __syncthreads();  // every read is done before the next round's writes
    }
  }
  if (MODE == RH_ROTATE) {
    if (a.inverse && a.signs) {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] *= a.signs_s[16 * p.cu + j];
    } else if (!a.signs) {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] *= a.scale;
    }
  } else if (a.inverse && a.signs) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= a.signs[16 * p.cu + j];
  }

  // ---- epilogue
  if (!QOUT) {
    if (p.live) store16(a.y, a.yt, p.row * a.ldy + p.col0, v);
    return;
  }
  // the quantizer of the output: the call's own, or the re-quantizer (absmax)
  constexpr int QB = MODE == RH_REQUANT ? BITS2 : BITS;
  constexpr int LVQ = (1 << QB) - 1;
  const int qkind = MODE == RH_REQUANT ? (int)BRQ_ABSMAX : a.qkind;
  const float qh = MODE == RH_REQUANT ? a.h2 : a.h;
  const int qgroup = MODE == RH_REQUANT ? a.group2 : a.group;
  uint8_t* const qcodes = a.codes + p.row * (MODE == RH_REQUANT ? a.codes_ld2 : a.codes_ld) + p.col0 * QB / 8;
  const int64_t qsidx = p.row * (MODE == RH_REQUANT ? a.scales_ld2 : a.scales_ld) + p.col0 / qgroup;
  // quantizer groups of g = 16 lpg consecutive columns are lpg consecutive lanes
  float stat = 0.f;
  if (qkind == BRQ_ABSMAX) {
#pragma unroll
    for (int j = 0; j < 16; ++j) stat = fmaxf(stat, fabsf(v[j]));
    stat = group_reduce<true>(stat, lpg);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) stat = fmaf(v[j], v[j], stat);
    stat = sqrtf(group_reduce<false>(stat, lpg));
  }
  if (R == 1 && bins) __syncthreads();  // the bin table (R > 1 passed barriers since)
  if (!p.live) return;
  // A zero group (stat 0, or not a number) codes as all zeros: its scale k is 0
  // and its offset puts every value on code 0.
  const bool nz = stat > 0.f;
  uint32_t c[16];
  if (qkind == BRQ_ABSMAX) {
    const float k = nz ? qh / stat : 0.f, off = nz ? qh : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = (int)rintf(fmaf(v[j], k, off));
      c[j] = (uint32_t)(q < 0 ? 0 : (q > LVQ ? LVQ : q));
    }
  } else if (MODE == RH_QUANT) {
    const float k = nz ? a.sqrt_g / stat : 0.f;
    // one branch for the whole thread: inside it the 16 table reads are
    // independent and pipeline
    if (bins) {
      // the decision in the bins' coordinate u = v k s + off, where the
      // table holds each threshold's own u; bin 0 holds no threshold
      const float ku = k * a.bin_s, off = nz ? a.bin_off : -1.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float u = fmaf(v[j], ku, off);
        const float2 e = tab[rh_bin(u)];
        c[j] = __float_as_uint(e.y) + (u > e.x ? 1u : 0u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float z = v[j] * k;
        int q = 0;
#pragma unroll
        for (int t = 0; t < LV; ++t) q += (z > a.tau[t]) ? 1 : 0;
        c[j] = nz ? (uint32_t)q : 0u;
      }
    }
  }
  store_codes<QB>(qcodes, c);
  if ((threadIdx.x & (lpg - 1)) == 0) {
    // quantize: v left out the transform's scale, so its statistic takes it
    const float st = MODE == RH_QUANT ? stat * a.scale : stat;
    if (qkind == BRQ_ABSMAX) static_cast<float*>(a.scales)[qsidx] = st;
    else static_cast<_Float16*>(a.scales)[qsidx] = (_Float16)st;
  }
}

template <int L2D, int MODE, int BITS, int BITS2 = 0>
hipError_t launch_t(const RhArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((rowhad_kernel<L2D, MODE, BITS, BITS2>), dim3((unsigned)rh_nwg(a)),
                     dim3(kRhThreads), 0, s, a);
  return hipGetLastError();
}

// The re-quantizer: output widths 2..5 for input widths 2..5, chunks of
// 64..256 (PolarQuant's blocks are 128).
template <int L2D, int BITS>
hipError_t launch_requant_out(const RhArgs& a, hipStream_t s) {
  switch (a.bits2) {
    case 2: return launch_t<L2D, RH_REQUANT, BITS, 2>(a, s);
    case 3: return launch_t<L2D, RH_REQUANT, BITS, 3>(a, s);
    case 4: return launch_t<L2D, RH_REQUANT, BITS, 4>(a, s);
    case 5: return launch_t<L2D, RH_REQUANT, BITS, 5>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int L2D>
hipError_t launch_requant(const RhArgs& a, hipStream_t s) {
  if constexpr (L2D >= 6 && L2D <= 8) {
    switch (a.bits) {
      case 2: return launch_requant_out<L2D, 2>(a, s);
      case 3: return launch_requant_out<L2D, 3>(a, s);
      case 4: return launch_requant_out<L2D, 4>(a, s);
      case 5: return launch_requant_out<L2D, 5>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int L2D, int MODE>
hipError_t launch_bits(const RhArgs& a, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_t<L2D, MODE, 2>(a, s);
    case 3: return launch_t<L2D, MODE, 3>(a, s);
    case 4: return launch_t<L2D, MODE, 4>(a, s);
    case 5: return launch_t<L2D, MODE, 5>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int L2D>
hipError_t launch_mode(const RhArgs& a, hipStream_t s) {
  if (a.mode == RH_ROTATE) return launch_t<L2D, RH_ROTATE, 0>(a, s);
  if (a.mode == RH_QUANT) return launch_bits<L2D, RH_QUANT>(a, s);
  if (a.mode == RH_REQUANT) return launch_requant<L2D>(a, s);
  return launch_bits<L2D, RH_DEQUANT>(a, s);
}

}  // namespace

hipError_t launch_rowhad(const RhArgs& a, hipStream_t s) {
  switch (a.log2d) {
    case 4: return launch_mode<4>(a, s);
    case 5: return launch_mode<5>(a, s);
    case 6: return launch_mode<6>(a, s);
    case 7: return launch_mode<7>(a, s);
    case 8: return launch_mode<8>(a, s);
    case 9: return launch_mode<9>(a, s);
    case 10: return launch_mode<10>(a, s);
    case 11: return launch_mode<11>(a, s);
    case 12: return launch_mode<12>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace brq
