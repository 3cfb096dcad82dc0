// MFMA kernels of the two-sided fast path (see fused.h for the decomposition).
//
// MFMA v_mfma_f32_16x16x4f32 lane layout (checked on gfx950): for lane l,
// lr = l % 16, lg = l / 16, the A operand is A[m = lr][k = lg], the B operand
// B[k = lg][n = lr], and result register i holds D[m = 4*lg + i][n = lr].
// Four steps over i with k = 4*lg + i contract 16 values.  Read as the A
// operand of the next product, D is the transpose: a stage that mixes the
// other index of the same 16 x 16 tile needs no data movement.
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

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }

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
    static_assert(PPW == 2, "float32 slabs hold two p per wave");
    v[0] = __uint_as_float(x.x);
    v[1] = __uint_as_float(x.y);
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

// The signs of both sides are folded into the stage-0 blocks at plan time, so
// the input is used as stored.  Per q: slab in (barrier), V_0 and U_0 on
// MFMA per 16-column output tile with the results into the output area
// (barrier), output area to global; the next slab is loaded into registers
// while the products run.  Loads and stores
// take one column c0 per wave instruction, so a lane's address is one
// loop-invariant register plus wave-uniform terms.
template <int ST, int WT>
__global__ __launch_bounds__(kFaWaves * 64, 1) void fused_a_kernel(FusedAArgs a) {
  constexpr int NB = fa_nb_of_steps(ST);
  constexpr int PPW = fa_ppw(WT, NB);
  constexpr int ESZ = fa_esz(WT);
  constexpr int P = 8 * PPW;
  constexpr int IPR = P * ESZ / 16;
  constexpr int KI = fa_ki(WT, ST);  // slab load instructions per wave
  constexpr int KQ = fa_kq_nt(WT, ST);  // output store instructions per wave and 16 columns
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = tid >> 6;
  const FaTile t = fa_tile(a, blockIdx.x, fa_nwg(a));
  const int bv = a.bv;
  const FaGeom g = fa_geom(WT, NB, bv);
  uint8_t* slab = smem;
  float* outa = reinterpret_cast<float*>(smem + g.slab_bytes);

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
      const FaSlot x = fa_slot(IPR, w, k, ln, bv, 0);
      const uint32_t off = (uint32_t)((x.r0 * 256 * a.ldw + x.c0 * 256 + (ln % IPR) * (16 / ESZ)) * ESZ);
      raw[k] = *reinterpret_cast<const uint4*>(base + off);
    }
  };

  // V_0 blocks of this wave's p: bvf[j][nt][s] = V[16 nt + lr][4 s + lg]
  float bvf[PPW][NB][ST];
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const float* vb = a.v0f + (int64_t)(t.p0 + PPW * w + j) * a.v0_gs;
#pragma unroll
    for (int nt = 0; nt < NB; ++nt)
#pragma unroll
      for (int sq = 0; 4 * sq < ST; ++sq) {
        const f4 v = ld4(vb + fa_vfrag(NB, nt, lr, lg, 4 * sq));
#pragma unroll
        for (int e = 0; e < 4 && 4 * sq + e < ST; ++e) bvf[j][nt][4 * sq + e] = v[e];
      }
  }
  int q = t.q0;
  load_slab(q);
  f4 bu = ld4(a.u0 + (int64_t)q * a.u0_gs + lr * 16 + 4 * lg);
  // nothing loaded before the loop is outstanding inside it, so the products
  // never wait on the prefetch of the next slab
  __builtin_amdgcn_s_waitcnt(0);

  for (int qi = 0; qi < kFaQC; ++qi, ++q) {
    // the previous slab's reads ended before the previous second barrier
    const int ls = opaque(lane);
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      const FaSlot x = fa_slot(IPR, w, k, ls, bv, 0);
      uint8_t* d = slab + fa_slab_item(g, x.r0, x.c0, ls % IPR);
      *reinterpret_cast<uint2*>(d) = make_uint2(raw[k].x, raw[k].y);
      *reinterpret_cast<uint2*>(d + 8) = make_uint2(raw[k].z, raw[k].w);
    }
    __syncthreads();  // slab complete
    const f4 bq = bu;
    uint8_t* obase = reinterpret_cast<uint8_t*>(a.ws) + ((int64_t)q * a.n + fa_col(a, t.chunk, 0, t.p0)) * 4;

    const uint8_t* arow = slab + fa_slab_read(g, lr, 0, w);
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      // V_0: D[j][m = r0][n = c0'] = sum_c0 X_j[r0][c0] V_j[c0'][c0], c0' = 16 nt + n.
      // The slab read of step s + 1 is issued before the products of step s.
      f4 d[PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) d[j] = f4{0.f, 0.f, 0.f, 0.f};
      uint2 nxt = fa_aread<WT, PPW>(arow + lg * g.rsb);
#pragma unroll
      for (int s = 0; s < ST; ++s) {
        const uint2 cur = nxt;
        if (s + 1 < ST) {
          const int c1 = 4 * (s + 1) + lg;  // only the last step can pass the radix
          nxt = fa_aread<WT, PPW>(arow + (s + 2 < ST || c1 < bv ? c1 : bv - 1) * g.rsb);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep that read ahead of this step's products
        const bool live = s + 1 < ST || 4 * s + lg < bv;
        float av[PPW];
        fa_unpack<WT, PPW>(cur, av);
#pragma unroll
        for (int j = 0; j < PPW; ++j) d[j] = mfma4(live ? av[j] : 0.f, bvf[j][nt][s], d[j]);
      }
      // the next slab's loads queue behind the previous stores: issued after
      // the first tile's products they no longer hold up the MFMA phase
      if (nt == 0 && qi + 1 < kFaQC) {
        load_slab(q + 1);
        bu = ld4(a.u0 + (int64_t)(q + 1) * a.u0_gs + lr * 16 + 4 * lg);
      }
      // U_0 on the transpose: E[j][m = c0'][n = r0'] = sum_r0 U[r0'][r0] D[j][r0][c0']
      f4 e[PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) e[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < PPW; ++j) e[j] = mfma4(d[j][i], bq[i], e[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 16 * nt + 4 * lg + i;
        if (c0 < bv) {
          float* o = outa + fa_out(g, lr, c0, PPW * w);
          if constexpr (PPW == 4)
            *reinterpret_cast<f4*>(o) = f4{e[0][i], e[1][i], e[2][i], e[3][i]};
          else
            *reinterpret_cast<float2*>(o) = make_float2(e[0][i], e[1][i]);
        }
      }
    }
    __syncthreads();  // output area complete; the slab may be overwritten

    const int lo = opaque(lane);
#pragma unroll
    for (int nt = 0; nt < NB; ++nt)
#pragma unroll
      for (int k = 0; k < KQ; ++k) {
        const FaSlot x = fa_slot(P / 4, w, k, lo, bv, 16 * nt);
        const int pq = lo % (P / 4);
        const f4 v = ld4(outa + fa_out(g, x.r0, x.c0, 4 * pq));
        *reinterpret_cast<f4*>(obase + (uint32_t)((x.r0 * 256 * a.n + x.c0 * 256 + 4 * pq) * 4)) = v;
      }
  }
}

// ------------------------------------------------------------------ pass B

// Group statistic of one lane's four values: absmax, or sum of squares for
// the norm quantizer (reduced over the four lane groups and rooted later).
template <int QK>
__device__ __forceinline__ float fb_stat(float acc, const f4& v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = QK == BRQ_ABSMAX ? fmaxf(acc, fabsf(v[i])) : fmaf(v[i], v[i], acc);
  return acc;
}

// Quantize and pack half h of the tile rows of r1.  The phase-2 results were
// written back in place into this wave's part of the exchange buffer, where
// slot (r1, c1h, r2, 4 lg) holds row r2's four consecutive columns
// c1 = 8h + c1h, c2 = 4 lg .. 4 lg + 3; stat[gi] holds this lane's part of
// group gi's statistic.  Each fragment is read back, coded and packed in turn.
template <int BITS, int QK, int G>
__device__ __forceinline__ void fb_quantize(const FusedBArgs& a, const FbTile& t, int r1, int h,
                                            const float* xch, const float (&stat_in)[128 / G], int lr,
                                            int lg) {
  constexpr int NG = 128 / G;      // groups in this half
  constexpr int FPG = 8 / NG;      // 16-column fragments per group
  constexpr int LV = (1 << BITS) - 1;
  constexpr int NW = FPG * 16 * BITS / 32;  // 32-bit code words per row and group
  const int64_t row = fb_row(t, r1, lr);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float stat = stat_in[gi];
    if (QK == BRQ_ABSMAX) {
      stat = fmaxf(stat, __shfl_xor(stat, 16, 64));
      stat = fmaxf(stat, __shfl_xor(stat, 32, 64));
    } else {
      stat += __shfl_xor(stat, 16, 64);
      stat += __shfl_xor(stat, 32, 64);
      stat = sqrtf(stat);
    }
    const float k = stat > 0.f ? (QK == BRQ_ABSMAX ? a.h / stat : a.sqrt_g / stat) : 0.f;
    // Packing: lane group lg assembles the words of fragments
    // [lg * FPG / 4, (lg + 1) * FPG / 4) when they end on a word boundary
    // (NW divisible by 4), else lane group 0 assembles all NW words.
    constexpr bool SPLIT = NW % 4 == 0;
    constexpr int NWL = SPLIT ? NW / 4 : NW;  // words per assembling lane
    uint32_t words[NWL];
#pragma unroll
    for (int j = 0; j < NWL; ++j) words[j] = 0u;
#pragma unroll
    for (int f = 0; f < FPG; ++f) {
      const f4 v = ld4(&xch[fb_xch(r1, gi * FPG + f, lr, 4 * lg)]);
      uint32_t c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int c = 0;
        if (stat > 0.f) {
          if (QK == BRQ_ABSMAX) {
            c = (int)__builtin_rintf(fmaf(v[i], k, a.h));
            c = c < 0 ? 0 : (c > LV ? LV : c);
          } else {
            const float z = v[i] * k;
#pragma unroll
            for (int q = 0; q < LV; ++q) c += (z > a.tau[q]) ? 1 : 0;
          }
        }
        c4 |= (uint32_t)c << (BITS * i);
      }
      // the row's four chunks of this fragment (4 codes each)
      const bool mine = SPLIT ? lg == f / (FPG / 4) : lg == 0;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t ch = (uint32_t)__shfl((int)c4, lr + 16 * q4, 64);
        const int bit = (SPLIT ? (f % (FPG / 4)) * 4 + q4 : f * 4 + q4) * 4 * BITS;
        const int wi = bit >> 5, sh = bit & 31;
        if (mine) {
          words[wi] |= ch << sh;
          if (sh + 4 * BITS > 32) words[wi + 1] |= ch >> (32 - sh);
        }
      }
      // one fragment at a time: read-ahead of the others would hold registers
      // that the prefetched tile needs
      __builtin_amdgcn_sched_barrier(0);
    }
    const int64_t col0 = fb_col(a, t, 8 * h + gi * FPG, 0);
    const int64_t gcol = col0 / G;
    if (lg == 0) {
      if (QK == BRQ_ABSMAX)
        static_cast<float*>(a.scales)[row * a.scales_ld + gcol] = stat;
      else
        static_cast<_Float16*>(a.scales)[row * a.scales_ld + gcol] = (_Float16)stat;
    }
    if (SPLIT || lg == 0) {
      uint32_t* out = reinterpret_cast<uint32_t*>(a.codes + row * a.codes_ld + col0 * BITS / 8) +
                      (SPLIT ? lg * NWL : 0);
#pragma unroll
      for (int j = 0; j < NWL; ++j) out[j] = words[j];
    }
  }
}

constexpr int FB_IL = 2;   // pass B phase 1: fragments whose MFMA chains interleave
constexpr int FB_IL2 = 2;  // pass B phase 2 (its registers are shared with the prefetched tile)

// Load half H of the tile's float32 block for phase 1: x[c2][i] = element
// (r1 = lr, c1 = 4 lg + i, r2 = w, c2) for i = 2H, 2H + 1, which is 128
// contiguous bytes of one row per lane.
template <int H>
__device__ __forceinline__ void fb_load_half(const FusedBArgs& a, const FbTile& t, int w, int lr,
                                             int lg, f4 (&x)[16]) {
  const float* src = a.ws + fb_row(t, lr, w) * a.n + fb_col(a, t, 4 * lg + 2 * H, 0);
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f4 v = ld4(src + e * 16 + 4 * qd);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * qd + j][2 * H + e] = v[j];
    }
}

// Persistent: workgroup b handles tiles b, b + gridDim.x, ...  Each half of
// the exchange frees half of every lane's tile registers, and the next
// tile's matching half is loaded into them at once, so the loads run under
// the second phase and the quantizer of the current tile.
template <int BITS, int QK, int G>
__global__ __launch_bounds__(kFbWaves * 64) void fused_b_kernel(FusedBArgs a) {
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

  f4 x[16];
  FbTile t = fb_tile(a, tile);
  fb_load_half<0>(a, t, w, lr, lg, x);
  fb_load_half<1>(a, t, w, lr, lg, x);
  f4 bu1 = ld4(a.u1 + (int64_t)(t.r0 * 16 + w) * a.u1_gs + lr * 16 + 4 * lg);
  f4 bu2 = ld4(a.u2 + (int64_t)(t.r0 * 16 + w) * a.u2_gs + lr * 16 + 4 * lg);

  for (;;) {
    __syncthreads();  // the previous tile is done with LDS
    // stage the tile's V_1 and V_2 blocks (16 each, groups c0*16 + f)
    for (int k = tid; k < 2 * 16 * 64; k += kFbWaves * 64) {
      const int which = k >> 10, rem = k & 1023, f = rem >> 6, qd = rem & 63;
      const float* src = (which ? a.v2 : a.v1) + (int64_t)(t.c0 * 16 + f) * (which ? a.v2_gs : a.v1_gs);
      *reinterpret_cast<f4*>(&lds[(which ? kFbV2Off : kFbV1Off) + f * 256 + 4 * qd]) = ld4(src + 4 * qd);
    }
    __syncthreads();

    // ---- phase 1: this wave owns r2 = w; fragments over (r1, c1), one per c2.
    lanes();
    const int v1_lane = kFbV1Off + fb_sigma(lr) * 16 + 4 * lg;
#pragma unroll
    for (int c2q = 0; c2q < 16; c2q += FB_IL) {
      f4 d[FB_IL];
#pragma unroll
      for (int f = 0; f < FB_IL; ++f) {
        // B[k = c1][n] = V_1[c1' = sigma(n)][c1]
        const f4 bv1 = ld4(&lds[v1_lane + (c2q + f) * 256]);
        d[f] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) d[f] = mfma4(x[c2q + f][i], bv1[i], d[f]);  // V_1: c1
        x[c2q + f] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < FB_IL; ++f) x[c2q + f] = mfma4(d[f][i], bu1[i], x[c2q + f]);  // U_1: r1
      // x[c2][j]: element (c1' = lg + 4 j, r1' = lr)
    }

    // ---- phase 2: this wave owns r1 = w; fragments over (r2, c2), one per c1.
    const int64_t next = tile + gridDim.x;
    // past the last tile, prefetch tile 0: every workgroup ending there reads
    // the same block, which then comes from cache instead of HBM
    const FbTile tn = fb_tile(a, next < ntiles ? next : 0);
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
          const int j = 2 * h + e;
          const f4 q4 = {x[4 * qd][j], x[4 * qd + 1][j], x[4 * qd + 2][j], x[4 * qd + 3][j]};
          *reinterpret_cast<f4*>(&xch[fb_xch(lro, lgo + 4 * e, w, 4 * qd)]) = q4;
        }
      // after the second half every tile register is free: load the whole
      // next tile (past the last one, tile 0, which keeps this code free of
      // branches)
      if (h == 1) {
        fb_load_half<0>(a, tn, w, lro, lgo, x);
        fb_load_half<1>(a, tn, w, lro, lgo, x);
      }
      __syncthreads();
      lanes();
      // only this wave reads the slots of r1 = w, so each result goes back
      // into the slot its input came from
      float stat[128 / G];
#pragma unroll
      for (int gi = 0; gi < 128 / G; ++gi) stat[gi] = 0.f;
#pragma unroll
      for (int c1q = 0; c1q < 8; c1q += FB_IL2) {
        f4 d[FB_IL2], v[FB_IL2];
#pragma unroll
        for (int f = 0; f < FB_IL2; ++f) {
          const f4 av = ld4(&xch[fb_xch(w, c1q + f, lr, 4 * lg)]);  // c2 = 4lg + i, r2 = lr
          const f4 bv2 = ld4(&lds[kFbV2Off + (8 * h + c1q + f) * 256 + lr * 16 + 4 * lg]);
          d[f] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) d[f] = mfma4(av[i], bv2[i], d[f]);  // V_2: c2
          v[f] = f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int f = 0; f < FB_IL2; ++f) v[f] = mfma4(d[f][i], bu2[i], v[f]);  // U_2: r2
        // v[f]: element (row r2' = lr, column c1 = 8h + c1q + f, c2' = 4lg + i)
#pragma unroll
        for (int f = 0; f < FB_IL2; ++f) {
          *reinterpret_cast<f4*>(&xch[fb_xch(w, c1q + f, lr, 4 * lg)]) = v[f];
          stat[(c1q + f) / (G / 16)] = fb_stat<QK>(stat[(c1q + f) / (G / 16)], v[f]);
        }
      }
      lanes();
      fb_quantize<BITS, QK, G>(a, t, w, h, xch, stat, lr, lg);
    }
    if (next >= ntiles) break;
    lanes();
    bu1 = ld4(a.u1 + (int64_t)(tn.r0 * 16 + w) * a.u1_gs + lr * 16 + 4 * lg);
    bu2 = ld4(a.u2 + (int64_t)(tn.r0 * 16 + w) * a.u2_gs + lr * 16 + 4 * lg);
    tile = next;
    t = tn;
  }
}

template <int ST, int WT>
hipError_t launch_a_t(const FusedAArgs& a, hipStream_t s) {
  static bool attr = false;  // output areas above 64 KiB of LDS need the opt-in
  if (!attr) {
    int most = 0;
    for (int bv = 4 * ST - 3; bv <= 4 * ST; ++bv) {
      const int b = fa_lds_bytes(fa_geom(WT, fa_nb_of_steps(ST), bv));
      most = b > most ? b : most;
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_a_kernel<ST, WT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, most);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const size_t lds = (size_t)fa_lds_bytes(fa_geom(WT, a.nb, a.bv));
  hipLaunchKernelGGL((fused_a_kernel<ST, WT>), dim3((unsigned)fa_nwg(a)), dim3(kFaWaves * 64), lds,
                     s, a);
  return hipGetLastError();
}

template <int ST>
hipError_t launch_a_st(const FusedAArgs& a, hipStream_t s) {
  if (a.wt == BRQ_F32) return launch_a_t<ST, BRQ_F32>(a, s);
  if (a.wt == BRQ_BF16) return launch_a_t<ST, BRQ_BF16>(a, s);
  return launch_a_t<ST, BRQ_F16>(a, s);
}

template <int... STs>
hipError_t launch_a_steps(const FusedAArgs& a, hipStream_t s, std::integer_sequence<int, STs...>) {
  hipError_t e = hipErrorInvalidValue;
  const int st = fa_steps(a.bv);
  ((st == STs + 1 ? (e = launch_a_st<STs + 1>(a, s), 0) : 0), ...);
  return e;
}

template <int BITS, int QK, int G>
hipError_t launch_b_t(const FusedBArgs& a, int grid, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_b_kernel<BITS, QK, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kFbLdsFloats * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((fused_b_kernel<BITS, QK, G>), dim3((unsigned)grid), dim3(kFbWaves * 64),
                     (size_t)kFbLdsFloats * sizeof(float), s, a);
  return hipGetLastError();
}

template <int BITS, int QK>
hipError_t launch_b_g(const FusedBArgs& a, int grid, hipStream_t s) {
  return a.group == 64 ? launch_b_t<BITS, QK, 64>(a, grid, s)
                       : launch_b_t<BITS, QK, 128>(a, grid, s);
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
