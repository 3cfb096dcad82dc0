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

// One input item: 8 consecutive p of one (r0, c0) segment.
template <int WT>
struct Raw {
  uint32_t v[WT == BRQ_F32 ? 8 : 4];
};

template <int WT>
__device__ __forceinline__ void fa_load_item(const FusedAArgs& a, const FaTile& t, int q, int it,
                                             Raw<WT>& r) {
  const int bv2 = a.bv * 2;
  const int r0 = it / bv2;
  const int rem = it - r0 * bv2;
  const int c0 = rem >> 1;
  const int hh = rem & 1;
  const int64_t row = fa_row(r0, q);
  const int64_t col = fa_col(a, t.chunk, c0, t.p0 + 8 * hh);
  if (WT == BRQ_F32) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.w) + row * a.ldw + col);
    const uint4 x0 = src[0], x1 = src[1];
    r.v[0] = x0.x; r.v[1] = x0.y; r.v[2] = x0.z; r.v[3] = x0.w;
    r.v[4] = x1.x; r.v[5] = x1.y; r.v[6] = x1.z; r.v[7] = x1.w;
  } else {
    const uint4 x0 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.w) + row * a.ldw + col);
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
__device__ __forceinline__ void fa_store_item(const FusedAArgs& a, const FaTile& t, int q, int it,
                                              const Raw<WT>& r, float* lds, int nb) {
  const int bv2 = a.bv * 2;
  const int r0 = it / bv2;
  const int rem = it - r0 * bv2;
  const int c0 = rem >> 1;
  const int hh = rem & 1;
  const float su = a.su ? a.su[fa_row(r0, q)] : 1.0f;
  const int cin = c0 * 256 + t.p0 + 8 * hh;  // column inside the chunk
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = fa_elem<WT>(r, e) * su;
    if (a.sv) v *= a.sv[cin + e];
    lds[fa_lds_in(nb, 8 * hh + e, r0, c0)] = v;
  }
}

template <int NB, int WT>
__global__ __launch_bounds__(kFaWaves * 64) void fused_a_kernel(FusedAArgs a) {
  extern __shared__ float lds[];
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

  const int items = 16 * bv * 2;  // <= 2048: at most two per thread
  Raw<WT> raw[2];
  int q = t.q0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int it = tid + k * kFaWaves * 64;
    if (it < items) fa_load_item<WT>(a, t, q, it, raw[k]);
  }

  for (int qi = 0; qi < kFaQC; ++qi, ++q) {
    __syncthreads();  // previous slice's LDS reads are done
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int it = tid + k * kFaWaves * 64;
      if (it < items) fa_store_item<WT>(a, t, q, it, raw[k], lds, NB);
    }
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
    // U_0 block of group q as B fragments: B[k = r0 = 4lg + i][n = r0' = lr] = U[lr][4lg + i]
    const f4 bu = ld4(a.u0 + (int64_t)q * a.u0_gs + lr * 16 + 4 * lg);
    if (qi + 1 < kFaQC) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int it = tid + k * kFaWaves * 64;
        if (it < items) fa_load_item<WT>(a, t, q + 1, it, raw[k]);
      }
    }
    __syncthreads();  // every wave holds its fragments; the slice may be overwritten

    // V_0: D[nt][m = r0][n = c0'] = sum_c0 X[r0][c0] V[c0'][c0]
    f4 d[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      d[nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) d[nt] = mfma4(af[kb][i], bvf[kb][nt][i], d[nt]);
    }
    // U_0 on the transpose: E[nt][m = c0'][n = r0'] = sum_r0 U[r0'][r0] D[r0][c0']
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      f4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) e = mfma4(d[nt][i], bu[i], e);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 16 * nt + 4 * lg + i;
        if (c0 < bv) lds[fa_lds_out(bv, lr, c0, w)] = e[i];
      }
    }
    __syncthreads();

    // store the slice: 16 x bv segments of kFaP floats, as float4
    const int quads = 16 * bv * (kFaP / 4);
    for (int it = tid; it < quads; it += kFaWaves * 64) {
      const int r0 = it / (bv * 4);
      const int rem = it - r0 * bv * 4;
      const int c0 = rem >> 2;
      const int qd = rem & 3;
      const f4 v = ld4(&lds[fa_lds_out(bv, r0, c0, 4 * qd)]);
      *reinterpret_cast<f4*>(a.ws + fa_row(r0, q) * a.n + fa_col(a, t.chunk, c0, t.p0 + 4 * qd)) = v;
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

template <int BITS, int QK, int G>
__global__ __launch_bounds__(kFbWaves * 64) void fused_b_kernel(FusedBArgs a) {
  extern __shared__ float xch[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = tid >> 6;
  const FbTile t = fb_tile(a, blockIdx.x);

  // ---- phase 1: this wave owns r2 = w; fragments over (r1, c1), one per c2.
  f4 x[16];  // x[c2][i] = element (r1 = lr, c1 = 4lg + i, r2 = w, c2)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float* src = a.ws + fb_row(t, lr, w) * a.n + fb_col(a, t, 4 * lg + i, 0);
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f4 v = ld4(src + 4 * qd);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * qd + j][i] = v[j];
    }
  }
  const f4 bu1 = ld4(a.u1 + (int64_t)(t.r0 * 16 + w) * a.u1_gs + lr * 16 + 4 * lg);
#pragma unroll
  for (int c2 = 0; c2 < 16; ++c2) {
    const f4 bv1 = ld4(a.v1 + (int64_t)(t.c0 * 16 + c2) * a.v1_gs + lr * 16 + 4 * lg);
    f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) d = mfma4(x[c2][i], bv1[i], d);  // V_1: mixes c1
    f4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) e = mfma4(d[i], bu1[i], e);      // U_1: mixes r1
    x[c2] = e;  // element (c1' = 4lg + i, r1' = lr)
  }

  // ---- phase 2: this wave owns r1 = w; fragments over (r2, c2), one per c1.
  const f4 bu2 = ld4(a.u2 + (int64_t)(t.r0 * 16 + w) * a.u2_gs + lr * 16 + 4 * lg);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
    if ((lg >> 1) == h) {
#pragma unroll
      for (int c2 = 0; c2 < 16; ++c2)
#pragma unroll
        for (int i = 0; i < 4; ++i) xch[fb_xch(lr, 4 * lg + i - 8 * h, w, c2)] = x[c2][i];
    }
    __syncthreads();
    f4 v[8];
#pragma unroll
    for (int c1h = 0; c1h < 8; ++c1h) {
      const f4 av = ld4(&xch[fb_xch(w, c1h, lr, 4 * lg)]);  // c2 = 4lg + i, r2 = lr
      const f4 bv2 = ld4(a.v2 + (int64_t)(t.c0 * 16 + 8 * h + c1h) * a.v2_gs + lr * 16 + 4 * lg);
      f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) d = mfma4(av[i], bv2[i], d);    // V_2: mixes c2
      f4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) e = mfma4(d[i], bu2[i], e);     // U_2: mixes r2
      v[c1h] = e;  // element (row r2' = lr, column c1 = 8h + c1h, c2' = 4lg + i)
    }
    fb_quantize<BITS, QK, G>(a, t, w, h, v, lr, lg);
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
hipError_t launch_b_t(const FusedBArgs& a, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_b_kernel<BITS, QK, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kFbXchFloats * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((fused_b_kernel<BITS, QK, G>), dim3((unsigned)fb_nwg(a)), dim3(kFbWaves * 64),
                     (size_t)kFbXchFloats * sizeof(float), s, a);
  return hipGetLastError();
}

template <int BITS, int QK>
hipError_t launch_b_g(const FusedBArgs& a, hipStream_t s) {
  return a.group == 64 ? launch_b_t<BITS, QK, 64>(a, s) : launch_b_t<BITS, QK, 128>(a, s);
}

template <int BITS>
hipError_t launch_b_k(const FusedBArgs& a, hipStream_t s) {
  return a.qkind == BRQ_ABSMAX ? launch_b_g<BITS, BRQ_ABSMAX>(a, s)
                               : launch_b_g<BITS, BRQ_CODEBOOK_NORM>(a, s);
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

hipError_t launch_fused_b(const FusedBArgs& a, hipStream_t s) {
  switch (a.bits) {
    case 2: return launch_b_k<2>(a, s);
    case 3: return launch_b_k<3>(a, s);
    case 4: return launch_b_k<4>(a, s);
    case 5: return launch_b_k<5>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace brq
