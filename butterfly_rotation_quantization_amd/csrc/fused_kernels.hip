// MFMA kernels of the two-sided fast path (see fused.h for the decomposition).
//
// MFMA v_mfma_f32_16x16x4f32 lane layout (checked on gfx950): for lane l,
// lr = l % 16, lg = l / 16, the A operand is A[m = lr][k = lg], the B operand
// B[k = lg][n = lr], and result register i holds D[m = 4*lg + i][n = lr].
// Four steps over i with k = 4*lg + i contract 16 values.  Read as the A
// operand of the next product, D is the transpose: a stage that mixes the
// other index of the same 16 x 16 tile needs no data movement.
//
// v_mfma_f32_16x16x32_f16 (pass B): lane l holds A[m = lr][k = 8 lg + s] and
// B[k = 8 lg + s][n = lr] in slot s = 0..7, and the result in the same layout
// as above (checked on gfx950, which also keeps f16 subnormal inputs).  Only
// the pairing of slots matters to the sum, so slot s < 4 carries k' = 4 lg + s
// of the 16-wide contraction and slot s >= 4 carries k' = 4 lg + s - 4 again,
// with the other half of a split operand: the lane's four accumulator values
// are still its A operand, and one instruction adds two split products.
//
// Stage arithmetic ([HARP] technical summary 2.1): every group of a stage is
// multiplied by its own b x b block, y_j = sum_k B[j][k] x_k; here the group
// index is fixed per tile and the batch of the product runs over the other
// matrix index, which shares the block.
#include <utility>

#include "fused.h"

namespace brq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));  // 16-byte aligned, as f4

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ void st4(float* p, const f4& v) { *reinterpret_cast<f4*>(p) = v; }

// The value itself, hidden from the optimizer: addresses derived from it are
// rebuilt where they are used instead of being hoisted out of a loop, where
// they would hold registers the tiles need.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float cvt_bf16(uint32_t w, int hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

__device__ __forceinline__ float cvt_f16(uint32_t w, int hi) {
  const uint16_t b = (uint16_t)(hi ? (w >> 16) : (w & 0xffffu));
  return (float)__builtin_bit_cast(_Float16, b);
}

// ------------------------------------------------------------------ split-f16 products

// One stage for one 16 x 16 fragment: the lane's four float32
// values a[i] (contraction index k = 4 lg + i) times the block entries for the
// same k, bhh = (bh, bh) and bll = (bl, bl).  The data split is hi = f16(a),
// lo = f16(a - hi), both rounded to nearest (a - hi is exact in float32, so
// hi + lo holds a to 2^-22 relative); products of f16 values are exact in
// float32.  m1 is -1 from a scalar register: a constant -1 would let the
// compiler turn the multiply-add into a subtraction, which costs a conversion
// of hi back to float32 where v_fma_mix_f32 reads the f16 directly.
//   (hi, lo) . (bh, bh), then (hi, lo) . (bl, bl) into the same accumulator
//   (not for blocks exact in f16, EX).
// The second product uses the same K = 32 instruction as the first: chained
// through the accumulator after a K = 32 product, v_mfma_f32_16x16x16_f16
// read a stale accumulator on gfx950 (the compiler issued them back to back).
template <bool EX>
__device__ __forceinline__ f4 fb_prod(const f4& a, const u4& bhh, const u4& bll, float m1) {
  const h4 hi = __builtin_convertvector(a, h4);
  f4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf((float)hi[i], m1, a[i]);
  const h4 lo = __builtin_convertvector(r, h4);
  const h8 A = __builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7);
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  const f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(h8, bhh), z, 0, 0, 0);
  if constexpr (EX) return d;
  else return __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(h8, bll), d, 0, 0, 0);
}

// -1 in a scalar register, hidden from constant folding.
__device__ __forceinline__ float fb_minus_one() {
  float v = -1.0f;
  asm volatile("" : "+s"(v));
  return v;
}

// (bh, bh) and (bl, bl) of a block entry (bh, bl).
__device__ __forceinline__ u4 fb_hh(const u4& e) { return u4{e.x, e.y, e.x, e.y}; }
__device__ __forceinline__ u4 fb_ll(const u4& e) { return u4{e.z, e.w, e.z, e.w}; }

// ------------------------------------------------------------------ pass A

// The ppw consecutive slab elements one lane reads per V_0 step: 8 bytes, or
// 4 for 16-bit input with ppw = 2 (then in .x).
template <int WT, int PPW>
__device__ __forceinline__ uint2 fa_aread(const uint8_t* src) {
  if constexpr (PPW * fa_esz(WT) == 8) return *reinterpret_cast<const uint2*>(src);
  else return make_uint2(*reinterpret_cast<const uint32_t*>(src), 0u);
}

template <int WT, int PPW>
__device__ __forceinline__ void fa_unpack(uint2 x, float (&v)[PPW]) {
  if constexpr (WT == BRQ_F32) {
    static_assert(PPW <= 2, "float32 slabs hold one or two p per wave");
    v[0] = __uint_as_float(x.x);
    if constexpr (PPW == 2) v[1] = __uint_as_float(x.y);
  } else if constexpr (PPW == 4) {
    if constexpr (WT == BRQ_BF16) {
      v[0] = cvt_bf16(x.x, 0); v[1] = cvt_bf16(x.x, 1);
      v[2] = cvt_bf16(x.y, 0); v[3] = cvt_bf16(x.y, 1);
    } else {
      v[0] = cvt_f16(x.x, 0); v[1] = cvt_f16(x.x, 1);
      v[2] = cvt_f16(x.y, 0); v[3] = cvt_f16(x.y, 1);
    }
  } else {
    if constexpr (WT == BRQ_BF16) {
      v[0] = cvt_bf16(x.x, 0); v[1] = cvt_bf16(x.x, 1);
    } else {
      v[0] = cvt_f16(x.x, 0); v[1] = cvt_f16(x.x, 1);
    }
  }
}

// The two 16-bit inputs of word w times 2^ks, as an f16 pair (the slab scale
// makes 16-bit inputs exact f16 values, so this is the operand the products
// take).
template <int WT>
__device__ __forceinline__ uint32_t fa_scaled_pair(uint32_t w, int ks) {
  const float a = WT == BRQ_BF16 ? cvt_bf16(w, 0) : cvt_f16(w, 0);
  const float b = WT == BRQ_BF16 ? cvt_bf16(w, 1) : cvt_f16(w, 1);
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const h2 r = __builtin_convertvector((f2{__builtin_ldexpf(a, ks), __builtin_ldexpf(b, ks)}), h2);
  return __builtin_bit_cast(uint32_t, r);
}

// Largest magnitude among the thread's slab items, as the bit pattern of a
// float32 (integer order equals magnitude order for finite values).
template <int WT, int KI>
__device__ __forceinline__ uint32_t fa_items_absmax(const uint4 (&raw)[KI]) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (WT == BRQ_F32) {
        const uint32_t v = wd[e] & 0x7fffffffu;
        m = v > m ? v : m;
      } else {
        const uint32_t lo = wd[e] & 0x7fffu, hi = (wd[e] >> 16) & 0x7fffu;
        const uint32_t v = lo > hi ? lo : hi;
        m = v > m ? v : m;
      }
    }
  }
  if constexpr (WT == BRQ_BF16) return m << 16;
  if constexpr (WT == BRQ_F16) return __float_as_uint((float)__builtin_bit_cast(_Float16, (uint16_t)m));
  return m;
}

// The signs of both sides are folded into the stage-0 blocks at plan time, so
// the input is used as stored.  Per q: slab in (barrier; with 16-bit inputs
// and more than one V_0 output tile, first the maxima (barrier), then the
// slab scaled and converted to f16 on its way into LDS), V_0 on MFMA output
// tile by output tile (chunk by chunk of 16 columns c0, the slab values read
// for each), U_0 per output tile with the results into the output area
// (barrier), output area to global; the next slab is loaded into registers
// while the products run.  Loads and stores take one column c0 per
// wave instruction, so a lane's address is one loop-invariant register plus
// wave-uniform terms.
template <int ST, int WT, int RU>
__global__ __launch_bounds__(kFaWaves * 64, 1) void fused_a_kernel(FusedAArgs a) {
  constexpr int NB = fa_nb_of_steps(ST);
  constexpr int MT = RU / 16;  // row tiles of the slab (r0 = 16 mt + lr)
  constexpr int PPW = fa_ppw(WT, NB);
  constexpr int ESZ = fa_esz(WT);
  constexpr int P = 8 * PPW;
  constexpr int IPR = P * ESZ / 16;
  constexpr int KI = fa_ki(WT, ST, RU);  // slab load instructions per wave
  constexpr int KQ = fa_kq_nt(WT, ST, RU);  // output store instructions per wave and 16 columns
  constexpr bool PRE = WT != BRQ_F32 && NB > 1;  // the slab holds scaled f16 operands
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = tid >> 6;
  const FaTile t = fa_tile(a, blockIdx.x, fa_nwg(a));
  const int bv = a.bv;
  const FaGeom g = fa_geom(WT, NB, bv, RU);
  uint8_t* slab = smem;
  float* outa = reinterpret_cast<float*>(smem + g.slab_bytes);
  uint32_t* smax = reinterpret_cast<uint32_t*>(smem + g.max_off);
  const float m1 = fb_minus_one();
  const int64_t ru_ld = (int64_t)a.su * a.ldw;  // input elements between rows r0 and r0 + 1
  const int64_t ru_n = (int64_t)a.su * a.n;     // output elements between rows r0 and r0 + 1

  // The per-instruction lane offsets are rebuilt from an opaque copy of the
  // lane index on every use: hoisted out of the q loop they would hold some
  // 30 registers that the V_0 blocks need.
  uint4 raw[KI];
  auto load_slab = [&](int q) {
    const uint8_t* base =
        static_cast<const uint8_t*>(a.w) + ((int64_t)q * a.ldw + fa_col(a, t.chunk, 0, t.p0)) * ESZ;
    const int ln = opaque(lane);
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      const FaSlot x = fa_slot(IPR, w, k, ln, bv, 0, RU);
      const uint32_t off = (uint32_t)((x.r0 * ru_ld + x.c0 * a.sv + (ln % IPR) * (16 / ESZ)) * ESZ);
      raw[k] = *reinterpret_cast<const uint4*>(base + off);
    }
  };
  // U_0 entries of q: eu[ot][kt] = (bh, bl) of U[16 ot + lr][16 kt + 4 lg + i]
  u4 eu[MT][MT];
  auto load_u = [&](int q) {
#pragma unroll
    for (int ot = 0; ot < MT; ++ot)
#pragma unroll
      for (int kt = 0; kt < MT; ++kt)
        eu[ot][kt] = *reinterpret_cast<const u4*>(a.u0 + (int64_t)q * a.u0_gs +
                                                  fa_uhentry(RU, 16 * ot + lr, 4 * kt + lg));
  };

  // V_0 entries of this wave's p: vb[j][nt][ch] = (bh, bl) of
  // V[16 nt + lr][16 ch + 4 lg + i]
  u4 vb[PPW][NB][NB];
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const uint16_t* vp = a.v0 + (int64_t)(t.p0 + PPW * w + j) * a.v0_gs;
#pragma unroll
    for (int nt = 0; nt < NB; ++nt)
#pragma unroll
      for (int ch = 0; ch < NB; ++ch)
        vb[j][nt][ch] = *reinterpret_cast<const u4*>(vp + fa_vhentry(NB, nt, lr, lg, ch));
  }
  int q = t.q0;
  load_slab(q);
  load_u(q);
  // nothing loaded before the loop is outstanding inside it, so the products
  // never wait on the prefetch of the next slab
  __builtin_amdgcn_s_waitcnt(0);

  for (int qi = 0; qi < a.qc; ++qi, ++q) {
    // the previous slab's reads ended before the previous second barrier
    {
      uint32_t mx = fa_items_absmax<WT, KI>(raw);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)mx, o, 64);
        mx = y > mx ? y : mx;
      }
      if (lane == 0) smax[w] = mx;
    }
    auto slab_scale = [&]() {
      uint32_t m = smax[0];
#pragma unroll
      for (int i = 1; i < kFaWaves; ++i) m = smax[i] > m ? smax[i] : m;
      return __builtin_amdgcn_readfirstlane(fa_scale_shift(m));
    };
    int ks = 0;
    const int ls = opaque(lane);
    // With several V_0 output tiles (radix above 16), 16-bit inputs go into
    // the slab already scaled and converted to f16, once, at the cost of a
    // barrier (the products read them for every output tile); otherwise, and
    // for float32 inputs, as loaded (converted, or split, where read)
    if constexpr (PRE) {
      __syncthreads();  // maxima complete
      ks = slab_scale();
    }
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      const FaSlot x = fa_slot(IPR, w, k, ls, bv, 0, RU);
      uint8_t* d = slab + fa_slab_item(g, x.r0, x.c0, ls % IPR);
      uint4 v = raw[k];
      if constexpr (PRE)
        v = make_uint4(fa_scaled_pair<WT>(v.x, ks), fa_scaled_pair<WT>(v.y, ks), fa_scaled_pair<WT>(v.z, ks),
                       fa_scaled_pair<WT>(v.w, ks));
      *reinterpret_cast<uint2*>(d) = make_uint2(v.x, v.y);
      *reinterpret_cast<uint2*>(d + 8) = make_uint2(v.z, v.w);
    }
    __syncthreads();  // slab (and, unless converted on the way in, maxima) complete
    if constexpr (!PRE) ks = slab_scale();
    u4 bhh[MT][MT], bll[MT][MT];
#pragma unroll
    for (int ot = 0; ot < MT; ++ot)
#pragma unroll
      for (int kt = 0; kt < MT; ++kt) {
        bhh[ot][kt] = fb_hh(eu[ot][kt]);
        bll[ot][kt] = fb_ll(eu[ot][kt]);
      }
    uint8_t* obase = reinterpret_cast<uint8_t*>(a.ws) + ((int64_t)q * a.n + fa_col(a, t.chunk, 0, t.p0)) * 4;

#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      // V_0: D[j][m = r0][n = c0'] = sum_c0 X_j[r0][c0] V_j[c0'][c0], c0' = 16 nt + n,
      // per row tile mt (r0 = 16 mt + m), one K = 32 product per 16 columns
      // c0: (hi, hi) . (bh, bl), and for float32 input also (lo, lo) . (bh, bl).
      // The lane's slab values x[r0][c0 = 16 ch + 4 lg + i] are read, scaled
      // and split per output tile (kept for all tiles they would need the
      // registers of the V_0 entries).
      f4 d[PPW][MT];
#pragma unroll
      for (int j = 0; j < PPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) d[j][mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint8_t* arow = slab + fa_slab_read(g, 16 * mt + lr, 0, w);
#pragma unroll
        for (int ch = 0; ch < NB; ++ch) {
          if constexpr (PRE) {
            // the lane's f16 operands x[r0][c0 = 16 ch + 4 lg + i] of its PPW
            // p: word j / 2 of read i holds p j in half j % 2
            uint2 rd[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c0 = 16 * ch + 4 * lg + i;
              const bool live = ch + 1 < NB || c0 < bv;
              rd[i] = fa_aread<WT, PPW>(arow + (live ? c0 : bv - 1) * g.rsb);
              if (!live) rd[i] = make_uint2(0u, 0u);
            }
#pragma unroll
            for (int j = 0; j < PPW; ++j) {
              const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
              const uint32_t w0 = __builtin_amdgcn_perm(j < 2 ? rd[1].x : rd[1].y, j < 2 ? rd[0].x : rd[0].y, sel);
              const uint32_t w1 = __builtin_amdgcn_perm(j < 2 ? rd[3].x : rd[3].y, j < 2 ? rd[2].x : rd[2].y, sel);
              const h4 hi = __builtin_bit_cast(h4, make_uint2(w0, w1));
              d[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_shufflevector(hi, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                __builtin_bit_cast(h8, vb[j][nt][ch]), d[j][mt], 0, 0, 0);
            }
            continue;
          }
          float xv[4][PPW];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c0 = 16 * ch + 4 * lg + i;
            const bool live = ch + 1 < NB || c0 < bv;  // only the last chunk can pass the radix
            const uint2 rd = fa_aread<WT, PPW>(arow + (live ? c0 : bv - 1) * g.rsb);
            fa_unpack<WT, PPW>(rd, xv[i]);
#pragma unroll
            for (int j = 0; j < PPW; ++j) xv[i][j] = live ? __builtin_ldexpf(xv[i][j], ks) : 0.f;
          }
#pragma unroll
          for (int j = 0; j < PPW; ++j) {
            const f4 xs = {xv[0][j], xv[1][j], xv[2][j], xv[3][j]};
            const h4 hi = __builtin_convertvector(xs, h4);
            d[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_shufflevector(hi, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                              __builtin_bit_cast(h8, vb[j][nt][ch]), d[j][mt], 0, 0, 0);
            if constexpr (WT == BRQ_F32) {
              f4 r;
#pragma unroll
              for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf((float)hi[i], m1, xs[i]);
              const h4 lo = __builtin_convertvector(r, h4);
              d[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_shufflevector(lo, lo, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                __builtin_bit_cast(h8, vb[j][nt][ch]), d[j][mt], 0, 0, 0);
            }
          }
        }
      }
      // the next slab's loads queue behind the previous stores: issued after
      // the last V_0 products they no longer hold up the MFMA phase
      if (nt == NB - 1 && qi + 1 < a.qc) {
        load_slab(q + 1);
        load_u(q + 1);
      }
      // U_0 on the transpose: E[j][m = c0'][n = r0'] = sum_r0 U[r0'][r0] D[j][r0][c0'],
      // r0' = 16 ot + n; each row tile kt of D is split once into (hi, lo)
      f4 e[PPW][MT];
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        h8 ad[MT];
#pragma unroll
        for (int kt = 0; kt < MT; ++kt) {
          const h4 hi = __builtin_convertvector(d[j][kt], h4);
          f4 r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf((float)hi[i], m1, d[j][kt][i]);
          ad[kt] = __builtin_shufflevector(hi, __builtin_convertvector(r, h4), 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int ot = 0; ot < MT; ++ot) {
          e[j][ot] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kt = 0; kt < MT; ++kt) {
            e[j][ot] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ad[kt], __builtin_bit_cast(h8, bhh[ot][kt]), e[j][ot],
                                                              0, 0, 0);
            if (!a.u0_exact)
              e[j][ot] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ad[kt], __builtin_bit_cast(h8, bll[ot][kt]),
                                                                e[j][ot], 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) e[j][ot][i] = __builtin_ldexpf(e[j][ot][i], -ks);
        }
      }
      // e[j][ot][i]: element (c0' = 16 nt + 4 lg + i, r0' = 16 ot + lr) of p j
#pragma unroll
      for (int ot = 0; ot < MT; ++ot)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c0 = 16 * nt + 4 * lg + i;
          if (c0 < bv) {
            float* o = outa + fa_out(g, 16 * ot + lr, c0, PPW * w);
            if constexpr (PPW == 4)
              *reinterpret_cast<f4*>(o) = f4{e[0][ot][i], e[1][ot][i], e[2][ot][i], e[3][ot][i]};
            else if constexpr (PPW == 2)
              *reinterpret_cast<float2*>(o) = make_float2(e[0][ot][i], e[1][ot][i]);
            else
              *o = e[0][ot][i];
          }
        }
    }
    __syncthreads();  // output area complete; the slab may be overwritten

    const int lo = opaque(lane);
#pragma unroll
    for (int nt = 0; nt < NB; ++nt)
#pragma unroll
      for (int k = 0; k < KQ; ++k) {
        const FaSlot x = fa_slot(P / 4, w, k, lo, bv, 16 * nt, RU);
        const int pq = lo % (P / 4);
        const f4 v = ld4(outa + fa_out(g, x.r0, x.c0, 4 * pq));
        *reinterpret_cast<f4*>(obase + (uint32_t)((x.r0 * ru_n + x.c0 * a.sv + 4 * pq) * 4)) = v;
      }
  }
}

// ------------------------------------------------------------------ pass B

// Quantize and pack half h of the tile rows of r1.  The phase-2 results were
// written back in place into this wave's part of the exchange buffer, slot
// (r1, c1h, r2, c2) holding row r2, column c1 = 8h + c1h, c2.  Lane (lr, lg)
// takes row r2 = lr and the 32 consecutive columns c1h = 2 lg, 2 lg + 1, all
// c2: it reduces their statistic, then with the lanes of the same row that
// share its quantizer group (lg ^ 1 for g = 64, all four lg for g = 128),
// codes the 32 values and writes them as BITS whole 32-bit words.  The values
// carry the tile scale 2^ks: the codes depend only on v / stat, which the
// power of two leaves exact, and the stored statistic is scaled back by
// 2^-ks (exact as well).
template <int BITS, int QK, int G>
__device__ __forceinline__ void fb_quantize(const FusedBArgs& a, const FbTile& t, int r1, int h,
                                            const float* xch, int lr, int lg, int ks) {
  constexpr int LV = (1 << BITS) - 1;
  // The values are read twice, for the statistic and for the codes: held
  // between the two they would take 32 registers next to the prefetched tile.
  float stat = 0.f;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const f4 v = ld4(&xch[fb_xch(r1, 2 * lg + (f >> 2), lr, 4 * (f & 3))]);
#pragma unroll
    for (int i = 0; i < 4; ++i) stat = QK == BRQ_ABSMAX ? fmaxf(stat, fabsf(v[i])) : fmaf(v[i], v[i], stat);
  }
  asm volatile("" ::: "memory");
  if (QK == BRQ_ABSMAX) {
    stat = fmaxf(stat, __shfl_xor(stat, 16, 64));
    if (G == 128) stat = fmaxf(stat, __shfl_xor(stat, 32, 64));
  } else {
    stat += __shfl_xor(stat, 16, 64);
    if (G == 128) stat += __shfl_xor(stat, 32, 64);
    stat = sqrtf(stat);
  }
  const bool live = stat > 0.f;  // a zero group codes as all zeros
  const float k = live ? (QK == BRQ_ABSMAX ? a.h / stat : a.sqrt_g / stat) : 0.f;
  // absmax: a zero group takes k = 0 and offset 0, so its codes come out 0
  // without a select per code
  const float off = live ? a.h : 0.f;
  uint32_t words[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) words[j] = 0u;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const f4 v = ld4(&xch[fb_xch(r1, 2 * lg + (f >> 2), lr, 4 * (f & 3))]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c;
      if (QK == BRQ_ABSMAX) {
        // |v| <= stat and k = RN(h / stat) keep v k + h within
        // [-h 2^-24, 2h (1 + 2^-24)], which rounds into [0, LV]: no clamp
        c = (int)__builtin_rintf(fmaf(v[i], k, off));
      } else {
        const float z = v[i] * k;
        c = 0;
#pragma unroll
        for (int q = 0; q < LV; ++q) c += (z > a.tau[q]) ? 1 : 0;
      }
      if (QK != BRQ_ABSMAX) c = live ? c : 0;
      const int bit = (4 * f + i) * BITS, wi = bit >> 5, sh = bit & 31;
      words[wi] |= (uint32_t)c << sh;
      if (sh + BITS > 32) words[wi + 1] |= (uint32_t)c >> (32 - sh);
    }
  }
  const int64_t row = fb_row(t, r1, lr);
  const int64_t col0 = fb_col(a, t, 8 * h + 2 * lg, 0);
  uint32_t* out = reinterpret_cast<uint32_t*>(a.codes + row * a.codes_ld + col0 * BITS / 8);
#pragma unroll
  for (int j = 0; j < BITS; ++j) out[j] = words[j];
  if (fb_scale_lane(lg, G)) {
    const int64_t gi = row * a.scales_ld + col0 / G;
    const float st = __builtin_ldexpf(stat, -ks);
    if (QK == BRQ_ABSMAX)
      static_cast<float*>(a.scales)[gi] = st;
    else
      static_cast<_Float16*>(a.scales)[gi] = (_Float16)st;
  }
}

constexpr int FB_IL = 2;   // pass B phase 1: fragments whose MFMA chains interleave
constexpr int FB_IL2 = 2;  // pass B phase 2 (its registers are shared with the prefetched tile)

// Load half H of the tile's float32 block for phase 1: x[c2] = elements
// (r1 = lr, c1 = 4 lg + 2H + e, r2 = w, c2) for e = 0, 1, which is 128
// contiguous bytes of one row per lane.  The tile is held as two arrays of
// float2 (c1 = 4 lg + {0, 1} and 4 lg + {2, 3}), so that each half's
// registers are free on their own once the exchange has taken them.
template <int H>
__device__ __forceinline__ void fb_load_half(const FusedBArgs& a, const FbTile& t, int w, int lr,
                                             int lg, float2 (&x)[16]) {
  const float* src = a.ws + fb_row(t, lr, w) * a.n + fb_col(a, t, 4 * lg + 2 * H, 0);
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f4 v = ld4(src + e * 16 + 4 * qd);
#pragma unroll
      for (int j = 0; j < 4; ++j) (e ? x[4 * qd + j].y : x[4 * qd + j].x) = v[j];
    }
}

// Persistent: workgroup b handles tiles b, b + gridDim.x, ...  Once the
// second half of the exchange has been written, every tile register is free
// and the next tile is loaded into them, so the loads run under the second
// half of phase 2 and its quantizer.
template <int BITS, int QK, int G, bool EX>
__global__ __launch_bounds__(kFbWaves * 64) void fused_b_kernel(FusedBArgs a) {
  static_assert(kFbWaves * 64 == 16 * 64, "one thread per entry of the 16 staged blocks of a stage");
  extern __shared__ float lds[];
  float* xch = lds;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Lane coordinates are re-derived from an opaque copy of the thread index
  // in every phase, so nothing computed from them lives across phases: the
  // tile and its prefetch need all but a few of the 128 registers.
  int lr, lg;
  auto lanes = [&]() {
    const int l = opaque(tid) & 63;
    lr = l & 15;
    lg = l >> 4;
  };
  lanes();
  const int64_t ntiles = fb_nwg(a);
  int64_t tile = blockIdx.x;
  if (tile >= ntiles) return;

  float2 xa[16], xb[16];
  FbTile t = fb_tile(a, tile);
  fb_load_half<0>(a, t, w, lr, lg, xa);
  fb_load_half<1>(a, t, w, lr, lg, xb);
  auto load_u = [&](const uint16_t* blk, int64_t gs, const FbTile& tt) {
    return *reinterpret_cast<const u4*>(blk + (int64_t)(tt.r0 * 16 + w) * gs + fb_hentry(lr, lg));
  };
  u4 e1 = load_u(a.u1, a.u1_gs, t), e2 = load_u(a.u2, a.u2_gs, t);
  const float m1 = fb_minus_one();

  for (;;) {
    // the tile's V_1 and V_2 block entries (16 blocks each, groups c0*16 + f):
    // thread tid stages entry tid of each, loaded before the wait for the tile
    u4 ve[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int f = tid >> 6, qd = tid & 63;
      ve[r] = *reinterpret_cast<const u4*>((r ? a.v2 : a.v1) + (int64_t)(t.c0 * 16 + f) * (r ? a.v2_gs : a.v1_gs) +
                                           fb_hentry(qd >> 2, qd & 3));
    }
    // the wave's largest magnitude (waits for the tile's loads)
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xa[c].x), fabsf(xa[c].y)), fmaxf(fabsf(xb[c].x), fabsf(xb[c].y))));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    __syncthreads();  // the previous tile is done with LDS
    if ((tid & 63) == 0) lds[kFbMaxOff + w] = mx;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int f = tid >> 6, j = (tid & 63) >> 2, q = tid & 3;
      st4(&lds[(r ? kFbV2Off : kFbV1Off) + f * 256 + fb_vslot(j, q)], __builtin_bit_cast(f4, fb_hh(ve[r])));
      if (!EX)
        st4(&lds[(r ? kFbV2LOff : kFbV1LOff) + f * 256 + fb_vslot(j, q)], __builtin_bit_cast(f4, fb_ll(ve[r])));
    }
    __syncthreads();
    // the tile scale 2^ks (uniform over the workgroup)
    int ks;
    {
      const f4 m0 = ld4(&lds[kFbMaxOff]), m1 = ld4(&lds[kFbMaxOff + 4]);
      const f4 m2 = ld4(&lds[kFbMaxOff + 8]), m3 = ld4(&lds[kFbMaxOff + 12]);
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fmaxf(m0[i], m1[i]), fmaxf(m2[i], m3[i])));
      ks = __builtin_amdgcn_readfirstlane(fb_scale_shift(__float_as_uint(m)));
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      xa[c] = make_float2(__builtin_ldexpf(xa[c].x, ks), __builtin_ldexpf(xa[c].y, ks));
      xb[c] = make_float2(__builtin_ldexpf(xb[c].x, ks), __builtin_ldexpf(xb[c].y, ks));
    }

    // ---- phase 1: this wave owns r2 = w; fragments over (r1, c1), one per c2.
    lanes();
    {
      const u4 bu1 = fb_hh(e1), bl1 = fb_ll(e1);
      const int v1_lane = kFbV1Off + fb_vslot(fb_sigma(lr), lg);
#pragma unroll
      for (int c2q = 0; c2q < 16; c2q += FB_IL) {
        f4 d[FB_IL];
#pragma unroll
        for (int f = 0; f < FB_IL; ++f) {
          // B[k = c1][n] = V_1[c1' = sigma(n)][c1]
          const u4 bv = __builtin_bit_cast(u4, ld4(&lds[v1_lane + (c2q + f) * 256]));
          const u4 bl = EX ? u4{0u, 0u, 0u, 0u}
                           : __builtin_bit_cast(u4, ld4(&lds[v1_lane + kFbV1LOff + (c2q + f) * 256]));
          const int c = c2q + f;
          d[f] = fb_prod<EX>(f4{xa[c].x, xa[c].y, xb[c].x, xb[c].y}, bv, bl, m1);  // V_1: c1
        }
#pragma unroll
        for (int f = 0; f < FB_IL; ++f) {
          const f4 r = fb_prod<EX>(d[f], bu1, bl1, m1);  // U_1: r1
          xa[c2q + f] = make_float2(r[0], r[1]);
          xb[c2q + f] = make_float2(r[2], r[3]);
        }
        // register j of fragment c2 (xa: j = 0, 1; xb: j = 2, 3): element
        // (c1' = lg + 4 j, r1' = lr)
      }
    }

    // ---- phase 2: this wave owns r1 = w; fragments over (r2, c2), one per c1.
    const int64_t next = tile + gridDim.x;
    const bool more = next < ntiles;  // uniform over the workgroup
    const FbTile tn = fb_tile(a, more ? next : tile);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lanes();
      const int lro = lr, lgo = lg;
      __syncthreads();  // phase 1 (h = 0) or the first half's reads (h = 1) are done
      // registers 2h and 2h + 1 hold c1' = lg + 8h and lg + 8h + 4; four
      // fragments give four consecutive c2 of one c1': one 16-byte write
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const float2* xh = h ? xb : xa;
          const f4 q4 = e ? f4{xh[4 * qd].y, xh[4 * qd + 1].y, xh[4 * qd + 2].y, xh[4 * qd + 3].y}
                          : f4{xh[4 * qd].x, xh[4 * qd + 1].x, xh[4 * qd + 2].x, xh[4 * qd + 3].x};
          *reinterpret_cast<f4*>(&xch[fb_xch(lro, lgo + 4 * e, w, 4 * qd)]) = q4;
        }
      // registers 2h and 2h + 1 are free now: load the next tile's half h
      // into them
      if (more) {
        if (h == 0) fb_load_half<0>(a, tn, w, lro, lgo, xa);
        else fb_load_half<1>(a, tn, w, lro, lgo, xb);
      }
      __syncthreads();
      lanes();
      // only this wave reads the slots of r1 = w, so each result goes back
      // into the slot its input came from
      const u4 bu2 = fb_hh(e2), bl2 = fb_ll(e2);
#pragma unroll
      for (int c1q = 0; c1q < 8; c1q += FB_IL2) {
        f4 d[FB_IL2];
#pragma unroll
        for (int f = 0; f < FB_IL2; ++f) {
          const f4 av = ld4(&xch[fb_xch(w, c1q + f, lr, 4 * lg)]);  // c2 = 4lg + i, r2 = lr
          const int c1 = 8 * h + c1q + f;
          const u4 bv = __builtin_bit_cast(u4, ld4(&lds[kFbV2Off + c1 * 256 + fb_vslot(lr, lg)]));
          const u4 bl = EX ? u4{0u, 0u, 0u, 0u}
                           : __builtin_bit_cast(u4, ld4(&lds[kFbV2LOff + c1 * 256 + fb_vslot(lr, lg)]));
          d[f] = fb_prod<EX>(av, bv, bl, m1);  // V_2: c2
        }
#pragma unroll
        for (int f = 0; f < FB_IL2; ++f) {
          const f4 v = fb_prod<EX>(d[f], bu2, bl2, m1);  // U_2: r2
          // v: element (row r2' = lr, column c1 = 8h + c1q + f, c2' = 4lg + i)
          *reinterpret_cast<f4*>(&xch[fb_xch(w, c1q + f, lr, 4 * lg)]) = v;
        }
      }
      // the quantizer reads what other lanes of this wave wrote: a wave's LDS
      // accesses complete in order, and the fence keeps the compiler from
      // moving the reads above the writes
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      lanes();
      fb_quantize<BITS, QK, G>(a, t, w, h, xch, lr, lg, ks);
    }
    if (!more) break;
    lanes();
    e1 = load_u(a.u1, a.u1_gs, tn);
    e2 = load_u(a.u2, a.u2_gs, tn);
    tile = next;
    t = tn;
  }
}

template <int ST, int WT, int RU>
hipError_t launch_a_t(const FusedAArgs& a, hipStream_t s) {
  static bool attr = false;  // output areas above 64 KiB of LDS need the opt-in
  if (!attr) {
    int most = 0;
    for (int bv = 4 * ST - 3; bv <= 4 * ST; ++bv) {
      const int b = fa_lds_bytes(fa_geom(WT, fa_nb_of_steps(ST), bv, RU));
      most = b > most ? b : most;
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_a_kernel<ST, WT, RU>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, most);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const size_t lds = (size_t)fa_lds_bytes(fa_geom(WT, a.nb, a.bv, RU));
  hipLaunchKernelGGL((fused_a_kernel<ST, WT, RU>), dim3((unsigned)fa_nwg(a)), dim3(kFaWaves * 64), lds,
                     s, a);
  return hipGetLastError();
}

template <int ST, int RU>
hipError_t launch_a_wt(const FusedAArgs& a, hipStream_t s) {
  if (a.wt == BRQ_F32) return launch_a_t<ST, BRQ_F32, RU>(a, s);
  if (a.wt == BRQ_BF16) return launch_a_t<ST, BRQ_BF16, RU>(a, s);
  return launch_a_t<ST, BRQ_F16, RU>(a, s);
}

// U_0 of radix 32 is built for V_0 radices up to 32 (two column chunks).
template <int ST>
hipError_t launch_a_st(const FusedAArgs& a, hipStream_t s) {
  if (a.ru == 16) return launch_a_wt<ST, 16>(a, s);
  if constexpr (ST <= 8) {
    if (a.ru == 32) return launch_a_wt<ST, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int... STs>
hipError_t launch_a_steps(const FusedAArgs& a, hipStream_t s, std::integer_sequence<int, STs...>) {
  hipError_t e = hipErrorInvalidValue;
  const int st = fa_steps(a.bv);
  ((st == STs + 1 ? (e = launch_a_st<STs + 1>(a, s), 0) : 0), ...);
  return e;
}

template <int BITS, int QK, int G, bool EX>
hipError_t launch_b_t(const FusedBArgs& a, int grid, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_b_kernel<BITS, QK, G, EX>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kFbLdsFloats * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((fused_b_kernel<BITS, QK, G, EX>), dim3((unsigned)grid), dim3(kFbWaves * 64),
                     (size_t)kFbLdsFloats * sizeof(float), s, a);
  return hipGetLastError();
}

template <int BITS, int QK, int G>
hipError_t launch_b_x(const FusedBArgs& a, int grid, hipStream_t s) {
  return a.exact ? launch_b_t<BITS, QK, G, true>(a, grid, s) : launch_b_t<BITS, QK, G, false>(a, grid, s);
}

template <int BITS, int QK>
hipError_t launch_b_g(const FusedBArgs& a, int grid, hipStream_t s) {
  return a.group == 64 ? launch_b_x<BITS, QK, 64>(a, grid, s)
                       : launch_b_x<BITS, QK, 128>(a, grid, s);
}

template <int BITS>
hipError_t launch_b_k(const FusedBArgs& a, int grid, hipStream_t s) {
  return a.qkind == BRQ_ABSMAX ? launch_b_g<BITS, BRQ_ABSMAX>(a, grid, s)
                               : launch_b_g<BITS, BRQ_CODEBOOK_NORM>(a, grid, s);
}

}  // namespace

hipError_t launch_fused_a(const FusedAArgs& a, hipStream_t s) {
  if (a.bv < 2 || a.bv > 64 || a.nb != fa_nb_of_steps(fa_steps(a.bv))) return hipErrorInvalidValue;
  return launch_a_steps(a, s, std::make_integer_sequence<int, 16>{});
}

hipError_t launch_fused_b(const FusedBArgs& a, int grid, hipStream_t s) {
  if (grid < 1 || grid > fb_nwg(a)) return hipErrorInvalidValue;
  switch (a.bits) {
    case 2: return launch_b_k<2>(a, grid, s);
    case 3: return launch_b_k<3>(a, grid, s);
    case 4: return launch_b_k<4>(a, grid, s);
    case 5: return launch_b_k<5>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace brq
