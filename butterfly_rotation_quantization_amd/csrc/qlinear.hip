// Quantized linear layer kernels (qlinear.h).
#include "qlinear.h"

#include <utility>

namespace brq {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

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

// Decoding.  A code q of b bits stands for the weight value 2q - L (L = 2^b
// - 1) times alpha / L.  The values are small odd integers, exact in f16 and
// bf16; they are made with bit operations and one exact multiply-add instead
// of integer-to-float conversions:
//  - f16: a 16-bit half whose mantissa holds q at bit o (o >= 1, o + b <= 10)
//    under the exponent of 1024 is the number 1024 + q 2^o; times 2^(1-o)
//    minus (2^(11-o) + L) it is 2q - L, and every step is exact.  Two codes
//    go into the halves of one word and one packed multiply-add finishes both.
//  - bf16: the same in float32 (exponent of 2^23, mantissa field at bit o,
//    1 <= o, o + b <= 23), then the upper halves of two floats are the bf16
//    values (small integers need at most 6 significant bits).
// The lane's codes of a group are a bit stream in words w[q] (stream bits
// [32q, 32q + 32)); sh[q] holds stream bits [32q + 16, 32q + 48).

// A two-byte window of the stream: register index (w: 0..NW-1, sh: NW..)
// and the byte offset of the window inside it.
struct QlWin {
  int reg, off;
};
template <int NW>
__host__ __device__ constexpr QlWin ql_win(int beta) {
  return beta % 4 <= 2 ? QlWin{beta / 4, beta % 4} : QlWin{NW + beta / 4, 1};
}

// (a & m) | c in one instruction (the compiler emits an and and an or when
// both constants are literals).
__device__ __forceinline__ uint32_t ql_and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

template <int NW>
__device__ __forceinline__ void ql_shifted(const uint32_t (&w)[NW], uint32_t (&sh)[NW]) {
#pragma unroll
  for (int q = 0; q < NW; ++q) sh[q] = __builtin_amdgcn_alignbit(q + 1 < NW ? w[q + 1] : 0u, w[q], 16);
}

template <int NW>
__device__ __forceinline__ uint32_t ql_reg(const uint32_t (&w)[NW], const uint32_t (&sh)[NW], int r) {
  return r < NW ? w[r] : sh[r - NW];
}

// f16 pair P of a lane's group: codes P (low half) and P + NC/2 (high half).
// The two codes sit NC b / 2 bits apart, a whole number of bytes, so they
// have the same bit offset in their windows and one byte permute brings both
// windows into one word.
template <int BITS, int NC, int P, bool FUSE>
__device__ __forceinline__ uint32_t ql_f16_pair(const uint32_t (&w)[(NC * BITS + 31) / 32],
                                                const uint32_t (&sh)[(NC * BITS + 31) / 32]) {
  constexpr int NW = (NC * BITS + 31) / 32, L = (1 << BITS) - 1;
  constexpr int a = P * BITS;
  constexpr int beta = a >= 1 ? (a - 1) / 8 : 0;  // the field starts at bit 1..8 of the window
  constexpr int o = a - 8 * beta;
  constexpr int betab = beta + (NC / 2) * BITS / 8;
  constexpr QlWin wa = ql_win<NW>(beta), wb = ql_win<NW>(betab);
  const uint32_t ra = ql_reg(w, sh, wa.reg), rb = ql_reg(w, sh, wb.reg);
  uint32_t d;
  if constexpr (wa.reg == wb.reg && wa.off == 0 && wb.off == 2) {
    d = ra;
  } else {
    constexpr uint32_t sel = (uint32_t)wa.off | (uint32_t)(wa.off + 1) << 8 | (uint32_t)(4 + wb.off) << 16 |
                             (uint32_t)(5 + wb.off) << 24;
    d = __builtin_amdgcn_perm(rb, ra, sel);
  }
  // field to bit o2 in [1, 10 - b]: a right shift moves high-half bits into
  // the top of the low half only (above the field); a left shift by one moves
  // the low half's top bit below the high field
  constexpr int o2 = o == 0 ? 1 : (o + BITS > 10 ? 10 - BITS : o);
  if constexpr (o2 > o) d <<= (o2 - o);
  else if constexpr (o2 < o) d >>= (o - o2);
  constexpr uint32_t m = ((1u << BITS) - 1u) << o2;
  const uint32_t v = FUSE ? ql_and_or(d, m | m << 16, 0x64006400u) : (d & (m | m << 16)) | 0x64006400u;
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  constexpr _Float16 c = (_Float16)(2.0f / (float)(1 << o2));
  constexpr _Float16 k = (_Float16)(-(float)((1 << (11 - o2)) + L));
  const h2v r = __builtin_bit_cast(h2v, v) * h2v{c, c} + h2v{k, k};
  return __builtin_bit_cast(uint32_t, r);
}

// float32 value 2q - L of code J (its field found in w, sh or w[0] << 8).
template <int BITS, int NC, int J, bool FUSE>
__device__ __forceinline__ float ql_f32_code(const uint32_t (&w)[(NC * BITS + 31) / 32],
                                             const uint32_t (&sh)[(NC * BITS + 31) / 32], uint32_t w0s) {
  constexpr int L = (1 << BITS) - 1;
  constexpr int a = J * BITS;
  constexpr int ow = a % 32, os = (a - 16) % 32;
  constexpr bool in_w = ow >= 1 && ow + BITS <= 23;
  constexpr bool in_s = a >= 16 && os >= 1 && os + BITS <= 23;
  constexpr int o = in_w ? ow : (in_s ? os : a + 8);
  static_assert(in_w || in_s || a + 8 + BITS <= 23, "no window for the code");
  uint32_t src;
  if constexpr (in_w) src = w[a / 32];
  else if constexpr (in_s) src = sh[(a - 16) / 32];
  else src = w0s;
  constexpr uint32_t m = ((1u << BITS) - 1u) << o;
  const float v = __uint_as_float(FUSE ? ql_and_or(src, m, 0x4B000000u) : (src & m) | 0x4B000000u);
  return fmaf(v, 2.0f / (float)(1 << o), -(float)((1 << (24 - o)) + L));
}

template <int BITS, int NC, bool FUSE, int... P>
__device__ __forceinline__ void ql_f16_pairs(const uint32_t (&w)[(NC * BITS + 31) / 32], uint32_t* out,
                                             std::integer_sequence<int, P...>) {
  uint32_t sh[(NC * BITS + 31) / 32];
  ql_shifted(w, sh);
  ((out[P] = ql_f16_pair<BITS, NC, P, FUSE>(w, sh)), ...);
}

template <int BITS, int NC, bool FUSE, int... P>
__device__ __forceinline__ void ql_bf16_pairs(const uint32_t (&w)[(NC * BITS + 31) / 32], uint32_t* out,
                                              std::integer_sequence<int, P...>) {
  uint32_t sh[(NC * BITS + 31) / 32];
  ql_shifted(w, sh);
  const uint32_t w0s = w[0] << 8;
  ((out[P] = __builtin_amdgcn_perm(__float_as_uint(ql_f32_code<BITS, NC, 2 * P + 1, FUSE>(w, sh, w0s)),
                                   __float_as_uint(ql_f32_code<BITS, NC, 2 * P, FUSE>(w, sh, w0s)), 0x07060302u)),
   ...);
}

// The products of one group: d[tm][tn] = sum over the group's inputs of the
// activations times the weight values 2q - L.  Lane group lg holds the
// inputs g0 + lg NC + [0, NC) (NC = G/4).  The order of the contraction
// inside a group is free as long as A and B follow the same one:
//  - f16: MFMA step s takes the pairs 4s + [0, 4) (pair p: inputs p and
//    p + NC/2), so the activations are interleaved in registers to match;
//  - bf16: step s takes inputs 8s .. 8s + 7 in order.
template <int BITS, bool BF, int G, int TM, int TN>
__device__ __forceinline__ void ql_group(f4v (&d)[TM][TN], const uint32_t (&wds)[TN][(G / 4 * BITS + 31) / 32],
                                         const uint16_t* const (&xrow)[TM], const bool (&tok_ok)[TM], int64_t g0) {
  constexpr int NC = G / 4;
  using V8 = typename std::conditional<BF, b8v, h8v>::type;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) d[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};
  uint32_t pr[TN][NC / 2];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    // the fused and-or helps the one- and two-tile kernels and costs the
    // four-tile ones registers
    if constexpr (BF) ql_bf16_pairs<BITS, NC, TM <= 2>(wds[tn], pr[tn], std::make_integer_sequence<int, NC / 2>{});
    else ql_f16_pairs<BITS, NC, TM <= 2>(wds[tn], pr[tn], std::make_integer_sequence<int, NC / 2>{});
  }
#pragma unroll
  for (int sp = 0; sp < NC / 16; ++sp) {  // two MFMA steps per activation load
    uint4 xa[TM], xb[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if constexpr (BF) {  // inputs 16 sp .. 16 sp + 15
        xa[tm] = tok_ok[tm] ? *reinterpret_cast<const uint4*>(xrow[tm] + g0 + 16 * sp) : make_uint4(0u, 0u, 0u, 0u);
        xb[tm] = tok_ok[tm] ? *reinterpret_cast<const uint4*>(xrow[tm] + g0 + 16 * sp + 8)
                            : make_uint4(0u, 0u, 0u, 0u);
      } else {  // inputs 8 sp + [0, 8) and the same plus NC/2
        xa[tm] = tok_ok[tm] ? *reinterpret_cast<const uint4*>(xrow[tm] + g0 + 8 * sp) : make_uint4(0u, 0u, 0u, 0u);
        xb[tm] = tok_ok[tm] ? *reinterpret_cast<const uint4*>(xrow[tm] + g0 + 8 * sp + NC / 2)
                            : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      V8 av[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        uint4 r;
        if constexpr (BF) {
          r = s2 == 0 ? xa[tm] : xb[tm];
        } else {  // pair p = 8 sp + 4 s2 + j: (x[p], x[p + NC/2]) from word 2 s2 + j/2, half j % 2
          const uint32_t a0 = s2 == 0 ? xa[tm].x : xa[tm].z, a1 = s2 == 0 ? xa[tm].y : xa[tm].w;
          const uint32_t b0 = s2 == 0 ? xb[tm].x : xb[tm].z, b1 = s2 == 0 ? xb[tm].y : xb[tm].w;
          r.x = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
          r.y = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
          r.z = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
          r.w = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
        }
        av[tm] = __builtin_bit_cast(V8, r);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int p0 = 8 * sp + 4 * s2;  // f16: pairs p0 .. p0 + 3; bf16: code pairs of inputs 2 p0 ..
        const uint4 braw = make_uint4(pr[tn][p0], pr[tn][p0 + 1], pr[tn][p0 + 2], pr[tn][p0 + 3]);
        const V8 bv = __builtin_bit_cast(V8, braw);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          if constexpr (BF) d[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tm], bv, d[tm][tn], 0, 0, 0);
          else d[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[tm], bv, d[tm][tn], 0, 0, 0);
        }
      }
    }
  }
}

// G: group size (64 or 128); TM: 16-token tiles per workgroup; TN: 16-output
// tiles per wave.  Each group loads the TM activation operands once for the
// TN output tiles and decodes each weight operand once for the TM token tiles
// (ql_group).
template <int BITS, bool BF, int G, int TM, int TN>
__global__ __launch_bounds__(kQlThreads) void qlinear_kernel(QlArgs a) {
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
    ql_group<BITS, BF, G, TM, TN>(d, wds, xrow, tok_ok, g0);
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

// Staging of one chunk for the streaming kernel: R weight rows x kQlChunk
// inputs of codes (16-byte pieces, consecutive threads along a row), their
// scales, and the tile's tv token rows of activations.
struct QlStage {
  const uint8_t* codes;  // the workgroup's first row
  int64_t codes_ld;
  const float* scales;
  int64_t scales_ld;
  const uint16_t* x;     // the tile's first token
  int64_t ldx;
  int tv;
};
template <int BITS, int G, int R, int TM, int CK = kQlChunk>
struct QlPieces {
  static constexpr int CB = CK * BITS / 8, NG = CK / G, XQ = CK / 8;
  static constexpr int NCP = R * (CB / 16) / kQlThreads, NSP = R * NG / kQlThreads;
  static constexpr int NXP = kQlTok * TM * XQ / kQlThreads;
};

template <int BITS, int G, int R, int TM, int CK = kQlChunk>
__device__ __forceinline__ void ql_fetch(const QlStage& st, int64_t k0, u4v (&pcod)[QlPieces<BITS, G, R, TM, CK>::NCP],
                                         float (&psc)[QlPieces<BITS, G, R, TM, CK>::NSP],
                                         u4v (&px)[QlPieces<BITS, G, R, TM, CK>::NXP]) {
  using P = QlPieces<BITS, G, R, TM, CK>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < P::NCP; ++i) {
    const int e = tid + i * kQlThreads, r = e / (P::CB / 16), q = e - r * (P::CB / 16);
    pcod[i] = *reinterpret_cast<const u4v*>(st.codes + r * st.codes_ld + k0 * BITS / 8 + 16 * q);
  }
#pragma unroll
  for (int i = 0; i < P::NSP; ++i) {
    const int e = tid + i * kQlThreads, r = e / P::NG, gq = e - r * P::NG;
    psc[i] = st.scales[r * st.scales_ld + k0 / G + gq];
  }
#pragma unroll
  for (int i = 0; i < P::NXP; ++i) {
    const int e = tid + i * kQlThreads, tk = e / P::XQ, q = e - tk * P::XQ;
    px[i] = tk < st.tv ? *reinterpret_cast<const u4v*>(st.x + tk * st.ldx + k0 + 8 * q) : u4v{0u, 0u, 0u, 0u};
  }
}

template <int BITS, int G, int R, int TM, int CK = kQlChunk>
__device__ __forceinline__ void ql_stash(int tv, float invL, uint8_t* lcodes, float* lscales, uint8_t* lx,
                                         const u4v (&pcod)[QlPieces<BITS, G, R, TM, CK>::NCP],
                                         const float (&psc)[QlPieces<BITS, G, R, TM, CK>::NSP],
                                         const u4v (&px)[QlPieces<BITS, G, R, TM, CK>::NXP]) {
  using P = QlPieces<BITS, G, R, TM, CK>;
  constexpr int PB = P::CB + 16, PS = P::NG + 1;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < P::NCP; ++i) {
    const int e = tid + i * kQlThreads, r = e / (P::CB / 16), q = e - r * (P::CB / 16);
    *reinterpret_cast<u4v*>(lcodes + r * PB + 16 * q) = pcod[i];
  }
#pragma unroll
  for (int i = 0; i < P::NSP; ++i) {
    const int e = tid + i * kQlThreads, r = e / P::NG, gq = e - r * P::NG;
    lscales[r * PS + gq] = psc[i] * invL;
  }
#pragma unroll
  for (int i = 0; i < P::NXP; ++i) {
    const int e = tid + i * kQlThreads, tk = e / P::XQ, q = e - tk * P::XQ;
    if (tk < tv) *reinterpret_cast<u4v*>(lx + tk * ql_xpitch(CK) + 16 * q) = px[i];
  }
}

// TM 16-token tiles with the loads of the next chunk in flight (kQlStream).
template <int BITS, bool BF, int G, int TM, int TN, bool ONE>
__global__ __launch_bounds__(kQlThreads) void qlinear_stream_kernel(QlArgs a) {
  constexpr int L = (1 << BITS) - 1;
  constexpr int NC = G / 4;
  constexpr int NW = (NC * BITS + 31) / 32;
  constexpr int R = kQlOut * TN;            // weight rows of the workgroup
  constexpr int CB = kQlChunk * BITS / 8;   // code bytes of a row per chunk
  constexpr int PB = CB + 16;               // LDS pitch
  constexpr int NG = kQlChunk / G;          // groups per chunk
  constexpr int PS = NG + 1;                // scale pitch (floats)
  constexpr int XQ = kQlChunk / 8;          // 16-byte pieces of a token's chunk
  // pieces per thread: codes, scales, activations (the divisions are exact)
  constexpr int NCP = R * (CB / 16) / kQlThreads;
  constexpr int NSP = R * NG / kQlThreads;
  constexpr int NXP = kQlTok * TM * XQ / kQlThreads;
  static_assert(NCP * kQlThreads == R * (CB / 16) && NSP * kQlThreads == R * NG &&
                    NXP * kQlThreads == kQlTok * TM * XQ,
                "staging pieces must divide among the threads");
  extern __shared__ __align__(16) uint8_t ql_lds[];
  uint8_t* lcodes = ql_lds;
  float* lscales = reinterpret_cast<float*>(ql_lds + R * PB);
  uint8_t* lx = ql_lds + R * PB + R * PS * 4;
  const QlTile t = ql_tile(a, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t row0 = t.ct * (int64_t)R;
  const int lrow0 = 16 * TN * w + lr;  // + 16 tn: this lane's rows within the workgroup
  const int64_t tok0 = t.tt * (int64_t)(kQlTok * TM);
  // tokens tok0 .. tok0 + tv - 1 exist
  const int tv = ONE ? 1 : (int)(a.T - tok0 < kQlTok * TM ? a.T - tok0 : kQlTok * TM);
  const int64_t k_beg = t.split * a.kc;
  const int64_t k_end = k_beg + a.kc < a.n ? k_beg + a.kc : a.n;
  const uint16_t* xrow[TM];
  bool tok_ok[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    xrow[tm] = reinterpret_cast<const uint16_t*>(lx + (16 * tm + lr) * kQlXPitch) + lg * NC;
    tok_ok[tm] = 16 * tm + lr < tv;
  }
  const float invL = 1.0f / (float)L;
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);

  u4v pcod[NCP];
  float psc[NSP];
  u4v px[NXP];
  const QlStage st{a.codes + row0 * a.codes_ld, a.codes_ld, a.scales + row0 * a.scales_ld, a.scales_ld,
                   xg + tok0 * a.ldx, a.ldx, tv};
  f4v acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};
  ql_fetch<BITS, G, R, TM>(st, k_beg, pcod, psc, px);  // k_end - k_beg is a positive multiple of kQlChunk
  for (int64_t k0 = k_beg; k0 < k_end; k0 += kQlChunk) {
    __syncthreads();  // the previous chunk's reads are done
    ql_stash<BITS, G, R, TM>(tv, invL, lcodes, lscales, lx, pcod, psc, px);
    __syncthreads();
    if (k0 + kQlChunk < k_end) ql_fetch<BITS, G, R, TM>(st, k0 + kQlChunk, pcod, psc, px);
#pragma unroll 2
    for (int gi = 0; gi < NG; ++gi) {
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
      ql_group<BITS, BF, G, TM, TN>(d, wds, xrow, tok_ok, (int64_t)gi * G);
      // D reg i holds token 16 tm + 4 lg + i: with one token only register 0 of lane group 0
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int i = 0; i < (ONE ? 1 : 4); ++i)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) acc[tm][tn][i] = fmaf(d[tm][tn][i], sc[tn], acc[tm][tn][i]);
    }
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 16 * tm + 4 * lg + i;
      if (tk < tv)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          a.part[((int64_t)t.split * a.T + tok0 + tk) * a.m + row0 + lrow0 + 16 * tn] = acc[tm][tn][i];
    }
}

template <int BITS, int G, bool BF>
__device__ __forceinline__ void ql_gemm_fetch(const QlStage& st, int64_t k0,
                                              u4v (&pcod)[QlGemmPieces<BITS, G, BF>::NCP],
                                              float (&psc)[QlGemmPieces<BITS, G, BF>::NSP],
                                              u4v (&px)[2 * QlGemmPieces<BITS, G, BF>::NXU]) {
  using P = QlGemmPieces<BITS, G, BF>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < P::NCP; ++i) {
    const int e = tid + i * P::NT, r = e / (P::CB / 16), q = e - r * (P::CB / 16);
    pcod[i] = *reinterpret_cast<const u4v*>(st.codes + r * st.codes_ld + k0 * BITS / 8 + 16 * q);
  }
#pragma unroll
  for (int i = 0; i < P::NSP; ++i) {
    const int e = tid + i * P::NT, r = e / P::NG, gq = e - r * P::NG;
    psc[i] = st.scales[r * st.scales_ld + k0 / G + gq];
  }
#pragma unroll
  for (int i = 0; i < P::NXU; ++i) {
    const int e = tid + i * P::NT, tk = e / P::UT, u = e - tk * P::UT;
    const uint16_t* xr = st.x + tk * st.ldx + k0;
    px[2 * i] = tk < st.tv ? *reinterpret_cast<const u4v*>(xr + P::nat0(u)) : u4v{0u, 0u, 0u, 0u};
    px[2 * i + 1] = tk < st.tv ? *reinterpret_cast<const u4v*>(xr + P::nat1(u)) : u4v{0u, 0u, 0u, 0u};
  }
}

template <int BITS, int G, bool BF>
__device__ __forceinline__ void ql_gemm_stash(int tv, float invL, uint8_t* lcodes, float* lscales, uint8_t* lx,
                                              const u4v (&pcod)[QlGemmPieces<BITS, G, BF>::NCP],
                                              const float (&psc)[QlGemmPieces<BITS, G, BF>::NSP],
                                              const u4v (&px)[2 * QlGemmPieces<BITS, G, BF>::NXU]) {
  using P = QlGemmPieces<BITS, G, BF>;
  constexpr int PB = P::CB + 16, PS = P::NG + 1, XP = ql_xpitch(P::CK);
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < P::NCP; ++i) {
    const int e = tid + i * P::NT, r = e / (P::CB / 16), q = e - r * (P::CB / 16);
    *reinterpret_cast<u4v*>(lcodes + r * PB + 16 * q) = pcod[i];
  }
#pragma unroll
  for (int i = 0; i < P::NSP; ++i) {
    const int e = tid + i * P::NT, r = e / P::NG, gq = e - r * P::NG;
    lscales[r * PS + gq] = psc[i] * invL;
  }
#pragma unroll
  for (int i = 0; i < P::NXU; ++i) {
    // every token row is written (rows past the last token with the zeros
    // the fetch left there), so the products read them unguarded
    const int e = tid + i * P::NT, tk = e / P::UT, u = e - tk * P::UT;
    {
      uint16_t* xr = reinterpret_cast<uint16_t*>(lx + tk * XP) + P::op0(u);
      const u4v a = px[2 * i], c = px[2 * i + 1];
      if constexpr (BF) {
        *reinterpret_cast<u4v*>(xr) = a;
        *reinterpret_cast<u4v*>(xr + 8) = c;
      } else {
        *reinterpret_cast<u4v*>(xr) =
            u4v{__builtin_amdgcn_perm(c.x, a.x, 0x05040100u), __builtin_amdgcn_perm(c.x, a.x, 0x07060302u),
                __builtin_amdgcn_perm(c.y, a.y, 0x05040100u), __builtin_amdgcn_perm(c.y, a.y, 0x07060302u)};
        *reinterpret_cast<u4v*>(xr + 8) =
            u4v{__builtin_amdgcn_perm(c.z, a.z, 0x05040100u), __builtin_amdgcn_perm(c.z, a.z, 0x07060302u),
                __builtin_amdgcn_perm(c.w, a.w, 0x05040100u), __builtin_amdgcn_perm(c.w, a.w, 0x07060302u)};
      }
    }
  }
}

// The products of one group for one 16-token tile: d[tn] = sum over the
// group's inputs of the activations (the tile's paired operands xo, two per
// 16 inputs) times the decoded weight operands pr (as ql_group makes them).
template <bool BF, int G, int TN>
__device__ __forceinline__ void ql_gemm_tile(f4v (&d)[TN], const uint32_t (&pr)[TN][G / 8], const uint4 (&xo)[G / 32]) {
  constexpr int NC = G / 4;
  using V8 = typename std::conditional<BF, b8v, h8v>::type;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) d[tn] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < NC / 16; ++sp) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const V8 av = __builtin_bit_cast(V8, xo[2 * sp + s2]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int p0 = 8 * sp + 4 * s2;
        const V8 bv = __builtin_bit_cast(V8, make_uint4(pr[tn][p0], pr[tn][p0 + 1], pr[tn][p0 + 2], pr[tn][p0 + 3]));
        if constexpr (BF) d[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, d[tn], 0, 0, 0);
        else d[tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, d[tn], 0, 0, 0);
      }
    }
  }
}

// A token tile's paired operands of one group: G/32 16-byte LDS reads.
template <int G>
__device__ __forceinline__ void ql_gemm_operands(uint4 (&xo)[G / 32], const uint16_t* xrow) {
#pragma unroll
  for (int j = 0; j < G / 32; ++j) xo[j] = *reinterpret_cast<const uint4*>(xrow + 8 * j);
}

// kQlGemm kernel.  Per group a wave decodes its two weight operands once and
// runs them against the eight token tiles; the next chunk is loaded into
// registers while the current one is multiplied.  The arithmetic per output
// is the streaming kernel's: each group's MFMA sum times alpha / L, added in
// group order.
template <int BITS, bool BF, int G>
__global__ __launch_bounds__(kQlGemmThreads, 1) void qlinear_gemm_kernel(QlArgs a) {
  using P = QlGemmPieces<BITS, G, BF>;
  constexpr int TM = kQlGemmTm, TN = kQlGemmTnw, CK = kQlGemmChunk, R = P::R;
  constexpr int L = (1 << BITS) - 1;
  constexpr int NC = G / 4;
  constexpr int NW = (NC * BITS + 31) / 32;
  constexpr int PB = P::CB + 16, PS = P::NG + 1, XP = ql_xpitch(CK);
  extern __shared__ __align__(16) uint8_t ql_lds[];
  uint8_t* lcodes = ql_lds;
  float* lscales = reinterpret_cast<float*>(ql_lds + R * PB);
  uint8_t* lx = ql_lds + R * PB + R * PS * 4;
  const QlTile t = ql_tile(a, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t row0 = t.ct * (int64_t)R;
  const int lrow0 = 16 * TN * w + lr;  // + 16 tn
  const int64_t tok0 = t.tt * (int64_t)(kQlTok * TM);
  const int tv = (int)(a.T - tok0 < kQlTok * TM ? a.T - tok0 : kQlTok * TM);
  const int64_t k_beg = t.split * a.kc;
  const int64_t k_end = k_beg + a.kc < a.n ? k_beg + a.kc : a.n;
  const float invL = 1.0f / (float)L;
  u4v pcod[P::NCP];
  float psc[P::NSP];
  u4v px[2 * P::NXU];
  const QlStage st{a.codes + row0 * a.codes_ld, a.codes_ld, a.scales + row0 * a.scales_ld, a.scales_ld,
                   static_cast<const uint16_t*>(a.x) + tok0 * a.ldx, a.ldx, tv};
  f4v acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f4v{0.f, 0.f, 0.f, 0.f};
  ql_gemm_fetch<BITS, G, BF>(st, k_beg, pcod, psc, px);  // k_end - k_beg is a positive multiple of CK
  for (int64_t k0 = k_beg; k0 < k_end; k0 += CK) {
    __syncthreads();  // the previous chunk's reads are done
    ql_gemm_stash<BITS, G, BF>(tv, invL, lcodes, lscales, lx, pcod, psc, px);
    __syncthreads();
    if (k0 + CK < k_end) ql_gemm_fetch<BITS, G, BF>(st, k0 + CK, pcod, psc, px);
#pragma unroll 1
    for (int gi = 0; gi < P::NG; ++gi) {
      uint32_t pr[TN][NC / 2];
      float sc[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        uint32_t wds[NW];
        const uint8_t* cp = lcodes + (lrow0 + 16 * tn) * PB + gi * (G * BITS / 8) + lg * (NC * BITS / 8);
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          if constexpr ((NC * BITS / 8) % 4 == 0) {
            wds[q] = reinterpret_cast<const uint32_t*>(cp)[q];
          } else {  // 2-byte aligned pieces
            const uint16_t* hp = reinterpret_cast<const uint16_t*>(cp);
            const int h0 = 2 * q;
            wds[q] = (uint32_t)hp[h0] | (h0 + 1 < NC * BITS / 16 ? (uint32_t)hp[h0 + 1] << 16 : 0u);
          }
        }
        if constexpr (BF) ql_bf16_pairs<BITS, NC, true>(wds, pr[tn], std::make_integer_sequence<int, NC / 2>{});
        else ql_f16_pairs<BITS, NC, true>(wds, pr[tn], std::make_integer_sequence<int, NC / 2>{});
        sc[tn] = lscales[(lrow0 + 16 * tn) * PS + gi];
      }
      // token tile tm's operands are read while tile tm - 1 is multiplied,
      // and tile tm - 1's sums are scaled after tile tm's products are
      // issued; the scheduling fences keep that order (left to itself the
      // compiler reuses one operand register for every read and waits on each)
      const uint16_t* xrow0 = reinterpret_cast<const uint16_t*>(lx + lr * XP) + gi * G + lg * NC;
      uint4 xo[G / 32], xn[G / 32];
      ql_gemm_operands<G>(xo, xrow0);
      f4v dp[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        if (tm + 1 < TM) ql_gemm_operands<G>(xn, xrow0 + (tm + 1) * (16 * XP / 2));
        f4v d[TN];
        ql_gemm_tile<BF, G, TN>(d, pr, xo);
        if (tm > 0)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[tm - 1][tn][i] = fmaf(dp[tn][i], sc[tn], acc[tm - 1][tn][i]);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) dp[tn] = d[tn];
#pragma unroll
        for (int j = 0; j < G / 32; ++j) xo[j] = xn[j];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[TM - 1][tn][i] = fmaf(dp[tn][i], sc[tn], acc[TM - 1][tn][i]);
    }
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 16 * tm + 4 * lg + i;
      if (tk < tv)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          a.part[((int64_t)t.split * a.T + tok0 + tk) * a.m + row0 + lrow0 + 16 * tn] = acc[tm][tn][i];
    }
}

__global__ void ql_reduce_kernel(const float* part, int splits, int64_t T, int64_t m, void* out,
                                 int ot, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * m) return;
  const int64_t t = i / m, o = i - t * m;
  // four running sums in a fixed order: part p goes to sum p mod 4.  The
  // parts are read 32 at a time, all loads of a batch in flight together
  // (a batch is one memory round trip; past the last part a slot adds 0).
  const int64_t st = T * m;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < splits; p += 32) {
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = p + j < splits ? part[(int64_t)(p + j) * st + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) s4[j & 3] += v[j];
  }
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
  if (a.kind == kQlGemm) {
    static bool attr = false;  // more than 64 KiB of LDS needs the opt-in
    if (!attr) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qlinear_gemm_kernel<BITS, BF, G>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)ql_gemm_lds_bytes(BITS, G, kQlTok * kQlGemmTm));
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL((qlinear_gemm_kernel<BITS, BF, G>), grid, dim3(kQlGemmThreads),
                       ql_gemm_lds_bytes(BITS, G, kQlTok * kQlGemmTm),
                       s, a);
  } else if (a.kind == kQlStream) {
    const size_t lds = ql_lds_bytes(BITS, G, kQlOut * kQlStreamTn, a.tv);
    if (a.tm == 2)
      hipLaunchKernelGGL((qlinear_stream_kernel<BITS, BF, G, 2, kQlStreamTn, false>), grid, dim3(kQlThreads), lds, s, a);
    else if (a.tv == 1)
      hipLaunchKernelGGL((qlinear_stream_kernel<BITS, BF, G, 1, kQlStreamTn, true>), grid, dim3(kQlThreads), lds, s, a);
    else
      hipLaunchKernelGGL((qlinear_stream_kernel<BITS, BF, G, 1, kQlStreamTn, false>), grid, dim3(kQlThreads), lds, s, a);
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
