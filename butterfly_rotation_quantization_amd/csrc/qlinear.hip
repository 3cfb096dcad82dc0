// Quantized linear layer kernels (qlinear.h).
#include "qlinear.h"

namespace brq {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));

// The codes of one lane for one group: g/4 consecutive codes of its weight
// row (inputs g0 + lg g/4 ...), gathered into 32-bit words (at most 5: 32
// codes of 5 bits).  Code i is bits [i BITS, (i + 1) BITS) of the words.
template <int BITS, int NC>
__device__ __forceinline__ void ql_chunk(const uint8_t* p, uint32_t (&wds)[(NC * BITS + 31) / 32]) {
  constexpr int NB = NC * BITS / 8;  // bytes: a whole number (NC is 16 or 32)
  constexpr int NW = (NC * BITS + 31) / 32;
  if constexpr (NB % 4 == 0) {
#pragma unroll
    for (int q = 0; q < NW; ++q) wds[q] = reinterpret_cast<const uint32_t*>(p)[q];
  } else {  // 2-byte aligned (NB even): 16-bit pieces
#pragma unroll
    for (int q = 0; q < NW; ++q) wds[q] = 0u;
#pragma unroll
    for (int h = 0; h < NB / 2; ++h)
      wds[h / 2] |= (uint32_t)reinterpret_cast<const uint16_t*>(p)[h] << (16 * (h & 1));
  }
}

template <int BITS, int NC>
__device__ __forceinline__ uint32_t ql_code(const uint32_t (&wds)[(NC * BITS + 31) / 32], int i) {
  const int bit = i * BITS, wi = bit >> 5, sh = bit & 31;
  uint32_t v = wds[wi] >> sh;
  if (sh + BITS > 32) v |= wds[wi + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

// G: group size (64 or 128); TM: 16-token tiles per workgroup; TN: 16-output
// tiles per wave.  Within a group, lane group lg takes the G/4 consecutive
// inputs g0 + lg G/4 + [0, G/4) and MFMA step s uses its inputs 8 s .. 8 s + 7
// (the contraction order inside the group is free, A and B follow the same
// one).  Each step loads the TM activation operands once for the TN output
// tiles and decodes each weight operand once for the TM token tiles.
template <int BITS, bool BF, int G, int TM, int TN>
__global__ __launch_bounds__(kQlThreads) void qlinear_kernel(QlArgs a) {
  using V8 = typename std::conditional<BF, b8v, h8v>::type;
  constexpr int L = (1 << BITS) - 1;
  constexpr int NC = G / 4;
  constexpr int NW = (NC * BITS + 31) / 32;
  const QlTile t = ql_tile(a, blockIdx.x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t ob = t.ct * ((int64_t)kQlOut * TN) + (int64_t)16 * TN * w + lr;  // + 16 tn
  const int64_t k_beg = t.split * a.kc;
  const int64_t k_end = k_beg + a.kc < a.n ? k_beg + a.kc : a.n;
  const uint16_t* xrow[TM];
  bool tok_ok[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t tok = (t.tt * TM + tm) * kQlTok + lr;  // this lane's token (A operand)
    tok_ok[tm] = tok < a.T;
    xrow[tm] = static_cast<const uint16_t*>(a.x) + (tok_ok[tm] ? tok : 0) * a.ldx + lg * NC;
  }
  const uint8_t* crow[TN];
  const float* srow[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    crow[tn] = a.codes + (ob + 16 * tn) * a.codes_ld + lg * NC * BITS / 8;
    srow[tn] = a.scales + (ob + 16 * tn) * a.scales_ld;
  }
  const float invL = 1.0f / (float)L;
  f4v acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int64_t g0 = k_beg; g0 < k_end; g0 += G) {
    uint32_t wds[TN][NW];
    float sc[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      ql_chunk<BITS, NC>(crow[tn] + g0 * BITS / 8, wds[tn]);
      sc[tn] = srow[tn][g0 / G] * invL;
    }
    f4v d[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) d[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NC / 8; ++st) {
      V8 av[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const uint4 raw = tok_ok[tm] ? *reinterpret_cast<const uint4*>(xrow[tm] + g0 + 8 * st)
                                     : make_uint4(0u, 0u, 0u, 0u);
        av[tm] = __builtin_bit_cast(V8, raw);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        V8 bv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int q = 2 * (int)ql_code<BITS, NC>(wds[tn], 8 * st + i) - L;
          if constexpr (BF) bv[i] = (__bf16)(float)q;
          else bv[i] = (_Float16)q;
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          if constexpr (BF) d[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tm], bv, d[tm][tn], 0, 0, 0);
          else d[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[tm], bv, d[tm][tn], 0, 0, 0);
        }
      }
    }
    // D reg i: token 4 lg + i of the tile, output lr: scale alpha(o, group) / L
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tm][tn][i] = fmaf(d[tm][tn][i], sc[tn], acc[tm][tn][i]);
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tk = (t.tt * TM + tm) * kQlTok + 4 * lg + i;
      if (tk < a.T)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          a.part[((int64_t)t.split * a.T + tk) * a.m + ob + 16 * tn] = acc[tm][tn][i];
    }
}

// The same product with the weight rows staged through LDS (qlinear.h).
template <int BITS, bool BF, int G, int TM, int TN>
__global__ __launch_bounds__(kQlThreads) void qlinear_staged_kernel(QlArgs a) {
  using V8 = typename std::conditional<BF, b8v, h8v>::type;
  constexpr int L = (1 << BITS) - 1;
  constexpr int NC = G / 4;
  constexpr int NW = (NC * BITS + 31) / 32;
  constexpr int R = kQlOut * TN;            // weight rows of the workgroup
  constexpr int CB = kQlChunk * BITS / 8;   // code bytes of a row per chunk
  constexpr int PB = CB + 16;               // LDS pitch
  constexpr int NG = kQlChunk / G;          // groups per chunk
  constexpr int PS = NG + 1;                // scale pitch (floats)
  extern __shared__ __align__(16) uint8_t ql_lds[];
  uint8_t* lcodes = ql_lds;
  float* lscales = reinterpret_cast<float*>(ql_lds + R * PB);
  const QlTile t = ql_tile(a, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t row0 = t.ct * (int64_t)R;
  const int lrow0 = 16 * TN * w + lr;  // + 16 tn: this lane's rows within the workgroup
  const int64_t k_beg = t.split * a.kc;
  const int64_t k_end = k_beg + a.kc < a.n ? k_beg + a.kc : a.n;
  const uint16_t* xrow[TM];
  bool tok_ok[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t tok = (t.tt * TM + tm) * kQlTok + lr;
    tok_ok[tm] = tok < a.T;
    xrow[tm] = static_cast<const uint16_t*>(a.x) + (tok_ok[tm] ? tok : 0) * a.ldx + lg * NC;
  }
  const float invL = 1.0f / (float)L;
  f4v acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = k_beg; k0 < k_end; k0 += kQlChunk) {  // k_end - k0 is a multiple of kQlChunk
    __syncthreads();  // the previous chunk's reads are done
    // codes: R rows x CB bytes in 16-byte pieces, consecutive threads along a row
    for (int pc = tid; pc < R * (CB / 16); pc += kQlThreads) {
      const int r = pc / (CB / 16), q = pc - r * (CB / 16);
      const uint4 v = *reinterpret_cast<const uint4*>(a.codes + (row0 + r) * a.codes_ld + k0 * BITS / 8 + 16 * q);
      *reinterpret_cast<uint4*>(lcodes + r * PB + 16 * q) = v;
    }
    for (int ps = tid; ps < R * NG; ps += kQlThreads) {
      const int r = ps / NG, gq = ps - r * NG;
      lscales[r * PS + gq] = a.scales[(row0 + r) * a.scales_ld + k0 / G + gq] * invL;
    }
    __syncthreads();
#pragma unroll 2
    for (int gi = 0; gi < NG; ++gi) {
      const int64_t g0 = k0 + (int64_t)gi * G;
      uint32_t wds[TN][NW];
      float sc[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const uint8_t* cp = lcodes + (lrow0 + 16 * tn) * PB + gi * (G * BITS / 8) + lg * (NC * BITS / 8);
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          if constexpr ((NC * BITS / 8) % 4 == 0) {
            wds[tn][q] = reinterpret_cast<const uint32_t*>(cp)[q];
          } else {  // 2-byte aligned pieces
            const uint16_t* hp = reinterpret_cast<const uint16_t*>(cp);
            const int h0 = 2 * q;
            wds[tn][q] = (uint32_t)hp[h0] | (h0 + 1 < NC * BITS / 16 ? (uint32_t)hp[h0 + 1] << 16 : 0u);
          }
        }
        sc[tn] = lscales[(lrow0 + 16 * tn) * PS + gi];
      }
      f4v d[TM][TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) d[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NC / 8; ++st) {
        V8 av[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const uint4 raw = tok_ok[tm] ? *reinterpret_cast<const uint4*>(xrow[tm] + g0 + 8 * st)
                                       : make_uint4(0u, 0u, 0u, 0u);
          av[tm] = __builtin_bit_cast(V8, raw);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          V8 bv;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int q = 2 * (int)ql_code<BITS, NC>(wds[tn], 8 * st + i) - L;
            if constexpr (BF) bv[i] = (__bf16)(float)q;
            else bv[i] = (_Float16)q;
          }
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) {
            if constexpr (BF) d[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tm], bv, d[tm][tn], 0, 0, 0);
            else d[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[tm], bv, d[tm][tn], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tm][tn][i] = fmaf(d[tm][tn][i], sc[tn], acc[tm][tn][i]);
    }
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tk = (t.tt * TM + tm) * kQlTok + 4 * lg + i;
      if (tk < a.T)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          a.part[((int64_t)t.split * a.T + tk) * a.m + row0 + lrow0 + 16 * tn] = acc[tm][tn][i];
    }
}

__global__ void ql_reduce_kernel(const float* part, int splits, int64_t T, int64_t m, void* out,
                                 int ot, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * m) return;
  const int64_t t = i / m, o = i - t * m;
  // four running sums in a fixed order (the loads of a round are independent)
  const int64_t st = T * m;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
  int p = 0;
  for (; p + 4 <= splits; p += 4)
#pragma unroll
    for (int j = 0; j < 4; ++j) s4[j] += part[(int64_t)(p + j) * st + i];
  for (; p < splits; ++p) s4[0] += part[(int64_t)p * st + i];
  const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
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

template <int BITS, bool BF, int G>
hipError_t launch_g(const QlArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)ql_blocks(a));
  const size_t lds = ql_lds_bytes(BITS, G, a.tm);
  if (a.staged) {
    if (a.tm == 4)
      hipLaunchKernelGGL((qlinear_staged_kernel<BITS, BF, G, 4, 2>), grid, dim3(kQlThreads), lds, s, a);
    else
      hipLaunchKernelGGL((qlinear_staged_kernel<BITS, BF, G, 1, 4>), grid, dim3(kQlThreads), lds, s, a);
  } else if (a.tm == 4) {
    hipLaunchKernelGGL((qlinear_kernel<BITS, BF, G, 4, 2>), grid, dim3(kQlThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((qlinear_kernel<BITS, BF, G, 1, 4>), grid, dim3(kQlThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_b(const QlArgs& a, hipStream_t s) {
  const bool bf = a.xt == BRQ_BF16;
  if (a.group == 64) return bf ? launch_g<BITS, true, 64>(a, s) : launch_g<BITS, false, 64>(a, s);
  if (a.group == 128) return bf ? launch_g<BITS, true, 128>(a, s) : launch_g<BITS, false, 128>(a, s);
  return hipErrorInvalidValue;
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
  hipLaunchKernelGGL(ql_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, s, part,
                     splits, T, m, out, ot, ldo);
  return hipGetLastError();
}

}  // namespace brq
