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
#include "fused.h"

namespace brq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }

__device__ __forceinline__ float cvt_bf16(uint32_t w, int hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

__device__ __forceinline__ float cvt_f16(uint32_t w, int hi) {
  const uint16_t b = (uint16_t)(hi ? (w >> 16) : (w & 0xffffu));
  return (float)__builtin_bit_cast(_Float16, b);
}

// ------------------------------------------------------------------ pass A

// One input item: the kFaP = 8 consecutive p of one (r0, c0) segment.
template <int WT>
struct Raw {
  uint32_t v[WT == BRQ_F32 ? 8 : 4];
};

template <int WT>
__device__ __forceinline__ void fa_load_item(const FusedAArgs& a, const FaTile& t, int q, int it,
                                             Raw<WT>& r) {
  const int r0 = fa_div_bv(a, it);
  const int c0 = it - r0 * a.bv;
  const int64_t off = fa_row(r0, q) * a.ldw + fa_col(a, t.chunk, c0, t.p0);
  if (WT == BRQ_F32) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.w) + off);
    const uint4 x0 = src[0], x1 = src[1];
    r.v[0] = x0.x; r.v[1] = x0.y; r.v[2] = x0.z; r.v[3] = x0.w;
    r.v[4] = x1.x; r.v[5] = x1.y; r.v[6] = x1.z; r.v[7] = x1.w;
  } else {
    const uint4 x0 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.w) + off);
    r.v[0] = x0.x; r.v[1] = x0.y; r.v[2] = x0.z; r.v[3] = x0.w;
  }
}

template <int WT>
__device__ __forceinline__ float fa_elem(const Raw<WT>& r, int e) {
  if (WT == BRQ_F32) return __uint_as_float(r.v[e]);
  if (WT == BRQ_BF16) return cvt_bf16(r.v[e >> 1], e & 1);
  return cvt_f16(r.v[e >> 1], e & 1);
}

template <int WT>
__device__ __forceinline__ void fa_store_item(const FusedAArgs& a, int it, const Raw<WT>& r,
                                              float* lds, int nb) {
  const int r0 = fa_div_bv(a, it);
  const int c0 = it - r0 * a.bv;
#pragma unroll
  for (int e = 0; e < kFaP; ++e) lds[fa_lds_in(nb, e, r0, c0)] = fa_elem<WT>(r, e);
}

// The signs of both sides are folded into the stage-0 blocks at plan time, so
// the input is used as stored.
template <int NB, int WT>
__global__ __launch_bounds__(kFaWaves * 64, 2) void fused_a_kernel(FusedAArgs a) {
  extern __shared__ float lds[];
  constexpr int NT = kFaWaves * 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = tid >> 6;  // this wave's p (local)
  const FaTile t = fa_tile(a, blockIdx.x, fa_nwg(a));
  const int bv = a.bv;
  const int p = t.p0 + w;

  // V_0 block of group p, as B fragments: bvf[kb][nt] = B[16nt + lr][16kb + 4lg + i]
  f4 bvf[NB][NB];
  {
    const float* vb = a.v0 + (int64_t)p * a.v0_gs;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int nt = 0; nt < NB; ++nt)
        bvf[kb][nt] = ld4(vb + (16 * nt + lr) * (16 * NB) + 16 * kb + 4 * lg);
  }

  const int items = 16 * bv;  // <= 1024: at most two per thread
  Raw<WT> raw[2];
  int q = t.q0;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (tid + k * NT < items) fa_load_item<WT>(a, t, q, tid + k * NT, raw[k]);
  // U_0 block of group q as B fragments: B[k = r0 = 4lg + i][n = r0' = lr] = U[lr][4lg + i]
  f4 bu = ld4(a.u0 + (int64_t)q * a.u0_gs + lr * 16 + 4 * lg);

  for (int qi = 0; qi < kFaQC; ++qi, ++q) {
    __syncthreads();  // previous slice's LDS reads are done
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (tid + k * NT < items) fa_store_item<WT>(a, tid + k * NT, raw[k], lds, NB);
    __syncthreads();

    // A fragments of X_qp: A[m = r0 = lr][k = c0 = 16kb + 4lg + i]
    f4 af[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      af[kb] = ld4(&lds[fa_lds_in(NB, w, lr, 16 * kb + 4 * lg)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * kb + 4 * lg + i >= bv) af[kb][i] = 0.f;
    }
    const f4 bu_q = bu;
    if (qi + 1 < kFaQC) {  // prefetch the next slice and its U_0 block
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (tid + k * NT < items) fa_load_item<WT>(a, t, q + 1, tid + k * NT, raw[k]);
      bu = ld4(a.u0 + (int64_t)(q + 1) * a.u0_gs + lr * 16 + 4 * lg);
    }
    __syncthreads();  // every wave holds its fragments; the slice may be overwritten

    // V_0: D[nt][m = r0][n = c0'] = sum_c0 X[r0][c0] V[c0'][c0]; the NB
    // accumulators are independent, so their products interleave.
    f4 d[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) d[nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) d[nt] = mfma4(af[kb][i], bvf[kb][nt][i], d[nt]);
    // U_0 on the transpose: E[nt][m = c0'][n = r0'] = sum_r0 U[r0'][r0] D[r0][c0']
    f4 e[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) e[nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < NB; ++nt) e[nt] = mfma4(d[nt][i], bu_q[i], e[nt]);
#pragma unroll
    for (int nt = 0; nt < NB; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 16 * nt + 4 * lg + i;
        if (c0 < bv) lds[fa_lds_out(bv, lr, c0, w)] = e[nt][i];
      }
    __syncthreads();

    // store the slice: 16 x bv runs of kFaP floats, as float4 pairs
    const int quads = items * (kFaP / 4);
    for (int it = tid; it < quads; it += NT) {
      const int rc = it >> 1, h2 = it & 1;
      const int r0 = fa_div_bv(a, rc);
      const int c0 = rc - r0 * bv;
      const f4 v = ld4(&lds[fa_lds_out(bv, r0, c0, 4 * h2)]);
      *reinterpret_cast<f4*>(a.ws + fa_row(r0, q) * a.n + fa_col(a, t.chunk, c0, t.p0 + 4 * h2)) = v;
    }
  }
}

// ------------------------------------------------------------------ pass B

template <int BITS, int QK, int G>
__device__ __forceinline__ void fb_quantize(const FusedBArgs& a, const FbTile& t, int r1, int h,
                                            const f4 (&v)[8], int lr, int lg) {
  constexpr int NG = 128 / G;      // groups in this half
  constexpr int FPG = 8 / NG;      // 16-column fragments per group
  constexpr int LV = (1 << BITS) - 1;
  const int64_t row = fb_row(t, r1, lr);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float stat = 0.f;
#pragma unroll
    for (int f = gi * FPG; f < (gi + 1) * FPG; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stat = QK == BRQ_ABSMAX ? fmaxf(stat, fabsf(v[f][i])) : fmaf(v[f][i], v[f][i], stat);
    if (QK == BRQ_ABSMAX) {
      stat = fmaxf(stat, __shfl_xor(stat, 16, 64));
      stat = fmaxf(stat, __shfl_xor(stat, 32, 64));
    } else {
      stat += __shfl_xor(stat, 16, 64);
      stat += __shfl_xor(stat, 32, 64);
      stat = sqrtf(stat);
    }
    const float k = stat > 0.f ? (QK == BRQ_ABSMAX ? a.h / stat : a.sqrt_g / stat) : 0.f;
    uint32_t chunk[FPG];
#pragma unroll
    for (int f = 0; f < FPG; ++f) {
      uint32_t c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = v[gi * FPG + f][i];
        int c = 0;
        if (stat > 0.f) {
          if (QK == BRQ_ABSMAX) {
            c = (int)__builtin_rintf(fmaf(x, k, a.h));
            c = c < 0 ? 0 : (c > LV ? LV : c);
          } else {
            const float z = x * k;
#pragma unroll
            for (int q = 0; q < LV; ++q) c += (z > a.tau[q]) ? 1 : 0;
          }
        }
        c4 |= (uint32_t)c << (BITS * i);
      }
      chunk[f] = c4;
    }
    const int64_t col0 = fb_col(a, t, 8 * h + gi * FPG, 0);
    const int64_t gcol = col0 / G;
    // gather the row's 4*FPG chunks (4 codes each) in lane group 0
    constexpr int NW = FPG * 16 * BITS / 32;
    uint32_t words[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) words[j] = 0u;
#pragma unroll
    for (int kk = 0; kk < FPG * 4; ++kk) {
      const uint32_t ch = (uint32_t)__shfl((int)chunk[kk >> 2], lr + 16 * (kk & 3), 64);
      const int bit = kk * 4 * BITS;
      const int wi = bit >> 5, sh = bit & 31;
      words[wi] |= ch << sh;
      if (sh + 4 * BITS > 32) words[wi + 1] |= ch >> (32 - sh);
    }
    if (lg == 0) {
      if (QK == BRQ_ABSMAX)
        static_cast<float*>(a.scales)[row * a.scales_ld + gcol] = stat;
      else
        static_cast<_Float16*>(a.scales)[row * a.scales_ld + gcol] = (_Float16)stat;
      uint32_t* out = reinterpret_cast<uint32_t*>(a.codes + row * a.codes_ld + col0 * BITS / 8);
#pragma unroll
      for (int j = 0; j < NW; ++j) out[j] = words[j];
    }
  }
}

constexpr int FB_IL = 2;  // pass B: fragments whose MFMA chains interleave

// Load the tile's float32 block for phase 1: x[c2][i] = element
// (r1 = lr, c1 = 4lg + i, r2 = w, c2), in quad-major order so the first
// fragments wait only for the first loads.
template <int QD0, int QD1>
__device__ __forceinline__ void fb_load_tile(const FusedBArgs& a, const FbTile& t, int w, int lr,
                                             int lg, f4 (&x)[16]) {
  const float* src = a.ws + fb_row(t, lr, w) * a.n + fb_col(a, t, 4 * lg, 0);
#pragma unroll
  for (int qd = QD0; qd < QD1; ++qd)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f4 v = ld4(src + i * 16 + 4 * qd);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * qd + j][i] = v[j];
    }
}

// Persistent: workgroup b handles tiles b, b + gridDim.x, ...; the next
// tile's data is loaded into registers while the current one finishes.
template <int BITS, int QK, int G>
__global__ __launch_bounds__(kFbWaves * 64) void fused_b_kernel(FusedBArgs a) {
  extern __shared__ float lds[];
  float* xch = lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = tid >> 6;
  const int64_t ntiles = fb_nwg(a);
  int64_t tile = blockIdx.x;
  if (tile >= ntiles) return;

  f4 x[16];
  FbTile t = fb_tile(a, tile);
  fb_load_tile<0, 2>(a, t, w, lr, lg, x);
  f4 bu1 = ld4(a.u1 + (int64_t)(t.r0 * 16 + w) * a.u1_gs + lr * 16 + 4 * lg);

  for (;;) {
    // fragments 0..7 were loaded ahead (with the previous tile); load 8..15
    fb_load_tile<2, 4>(a, t, w, lr, lg, x);
    const f4 bu2 = ld4(a.u2 + (int64_t)(t.r0 * 16 + w) * a.u2_gs + lr * 16 + 4 * lg);
    __syncthreads();  // the previous tile is done with LDS
    // stage the tile's V_1 and V_2 blocks (16 each, groups c0*16 + f)
    for (int k = tid; k < 2 * 16 * 64; k += kFbWaves * 64) {
      const int which = k >> 10, rem = k & 1023, f = rem >> 6, qd = rem & 63;
      const float* src = (which ? a.v2 : a.v1) + (int64_t)(t.c0 * 16 + f) * (which ? a.v2_gs : a.v1_gs);
      *reinterpret_cast<f4*>(&lds[(which ? kFbV2Off : kFbV1Off) + f * 256 + 4 * qd]) = ld4(src + 4 * qd);
    }
    __syncthreads();

    // ---- phase 1: this wave owns r2 = w; fragments over (r1, c1), one per c2.
#pragma unroll
    for (int c2q = 0; c2q < 16; c2q += FB_IL) {
      f4 d[FB_IL];
#pragma unroll
      for (int f = 0; f < FB_IL; ++f) {
        const f4 bv1 = ld4(&lds[kFbV1Off + (c2q + f) * 256 + lr * 16 + 4 * lg]);
        d[f] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) d[f] = mfma4(x[c2q + f][i], bv1[i], d[f]);  // V_1: c1
        x[c2q + f] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < FB_IL; ++f) x[c2q + f] = mfma4(d[f][i], bu1[i], x[c2q + f]);  // U_1: r1
      // x[c2]: element (c1' = 4lg + i, r1' = lr)
    }

    // ---- phase 2: this wave owns r1 = w; fragments over (r2, c2), one per c1.
    const int64_t next = tile + gridDim.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
      if ((lg >> 1) == h) {
        // four fragments give four consecutive c2 of one c1: one 16-byte write
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f4 q4 = {x[4 * qd][i], x[4 * qd + 1][i], x[4 * qd + 2][i], x[4 * qd + 3][i]};
            *reinterpret_cast<f4*>(&xch[fb_xch(lr, 4 * lg + i - 8 * h, w, 4 * qd)]) = q4;
          }
      }
      if (h == 1 && next < ntiles) {  // x is free: prefetch half of the next tile
        const FbTile tn = fb_tile(a, next);
        fb_load_tile<0, 2>(a, tn, w, lr, lg, x);
        bu1 = ld4(a.u1 + (int64_t)(tn.r0 * 16 + w) * a.u1_gs + lr * 16 + 4 * lg);
      }
      __syncthreads();
      f4 v[8];
#pragma unroll
      for (int c1q = 0; c1q < 8; c1q += FB_IL) {
        f4 d[FB_IL];
#pragma unroll
        for (int f = 0; f < FB_IL; ++f) {
          const f4 av = ld4(&xch[fb_xch(w, c1q + f, lr, 4 * lg)]);  // c2 = 4lg + i, r2 = lr
          const f4 bv2 = ld4(&lds[kFbV2Off + (8 * h + c1q + f) * 256 + lr * 16 + 4 * lg]);
          d[f] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) d[f] = mfma4(av[i], bv2[i], d[f]);  // V_2: c2
          v[c1q + f] = f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int f = 0; f < FB_IL; ++f) v[c1q + f] = mfma4(d[f][i], bu2[i], v[c1q + f]);  // U_2: r2
      }
      // v[c1h]: element (row r2' = lr, column c1 = 8h + c1h, c2' = 4lg + i)
      fb_quantize<BITS, QK, G>(a, t, w, h, v, lr, lg);
    }
    if (next >= ntiles) break;
    tile = next;
    t = fb_tile(a, tile);
  }
}

template <int NB, int WT>
hipError_t launch_a_t(const FusedAArgs& a, hipStream_t s) {
  static bool attr = false;  // slices above 64 KiB of LDS need the opt-in
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_a_kernel<NB, WT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       fa_lds_floats(NB, 16 * NB) * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr = true;
  }
  const size_t lds = (size_t)fa_lds_floats(NB, a.bv) * sizeof(float);
  hipLaunchKernelGGL((fused_a_kernel<NB, WT>), dim3((unsigned)fa_nwg(a)), dim3(kFaWaves * 64), lds,
                     s, a);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_a_nb(const FusedAArgs& a, hipStream_t s) {
  if (a.wt == BRQ_F32) return launch_a_t<NB, BRQ_F32>(a, s);
  if (a.wt == BRQ_BF16) return launch_a_t<NB, BRQ_BF16>(a, s);
  return launch_a_t<NB, BRQ_F16>(a, s);
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
  switch (a.nb) {
    case 1: return launch_a_nb<1>(a, s);
    case 2: return launch_a_nb<2>(a, s);
    case 3: return launch_a_nb<3>(a, s);
    case 4: return launch_a_nb<4>(a, s);
  }
  return hipErrorInvalidValue;
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
