// Stage pass kernel: one stage of one side over the whole matrix (stage.h).
#include "stage.h"

namespace brq {
namespace {

__device__ __forceinline__ float sp_load(const void* p, int t, int64_t i) {
  if (t == BRQ_F32) return static_cast<const float*>(p)[i];
  if (t == BRQ_BF16)
    return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  return (float)static_cast<const _Float16*>(p)[i];
}

__device__ __forceinline__ void sp_store(void* p, int t, int64_t i, float v) {
  if (t == BRQ_F32) {
    static_cast<float*>(p)[i] = v;
  } else if (t == BRQ_BF16) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) u |= 0x400000u;  // keep NaN a quiet NaN
    else u += 0x7fffu + ((u >> 16) & 1u);                   // nearest, ties to even
    static_cast<uint16_t*>(p)[i] = (uint16_t)(u >> 16);
  } else {
    static_cast<_Float16*>(p)[i] = (_Float16)v;
  }
}

template <int MAXB, int SIDE, int LINES>
__global__ __launch_bounds__(kSpThreads) void stage_kernel(SpArgs a) {
  // one tile buffer: the outputs wait in registers until every input is read
  __shared__ __align__(16) float buf[SIDE ? kSpBufFloats : LINES * kSpLineFloats];
  __shared__ int spos[kSpLineFloats];   // left side: position of tile member q (-1: none)
  __shared__ int sslot[kSpLineFloats];  // left side: its LDS slot at line 0 (+ l for line l)
  const int u = threadIdx.x;
  int64_t gt, lt;
  sp_tile_of_block(a, blockIdx.x, gt, lt);
  const int64_t g0 = gt * a.gw;
  const int64_t l0 = lt * LINES;
  const int ng = (int)(a.ngroups - g0 < a.gw ? a.ngroups - g0 : a.gw);
  const int nl = (int)(a.lines - l0 < LINES ? a.lines - l0 : LINES);
  const int gb = a.gw * a.b;
  constexpr int kStep = kSpThreads / LINES;  // left side: members per pass over the lines

  // ---- tile in.  Right side: thread u owns member u and walks the lines.
  // Left side: thread u owns line u % 32 and members u / 32 + 8 it, whose
  // positions come from a table built once per tile.
  float v[LINES];
  int mg = 0, mk = 0;
  int64_t mpos = 0;
  float sg_out = 1.f;  // right side: the member's output sign, loaded with its inputs
  if (a.side == 0) {
    if (u < gb) {
      sp_member(a, u, mg, mk);
      if (mg < ng) {
        mpos = sp_pos(a, g0 + mg, mk);
        if (a.nparts > 1) {  // the sum of the parts, in their fixed order
#pragma unroll
          for (int l = 0; l < LINES; ++l) {
            if (l < nl) {
              const float* src = static_cast<const float*>(a.src) + sp_off(a, l0 + l, mpos, a.ld_src);
              // eight parts at a time, all eight loads in flight (past the
              // last part a slot adds 0)
              float s4[4] = {0.f, 0.f, 0.f, 0.f};
              for (int p0 = 0; p0 < a.nparts; p0 += 8) {
                float v8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v8[j] = p0 + j < a.nparts ? src[(int64_t)(p0 + j) * a.part_stride] : 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) s4[j & 3] += v8[j];
              }
              v[l] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            }
          }
        } else {
#pragma unroll
          for (int l = 0; l < LINES; ++l)
            if (l < nl) v[l] = sp_load(a.src, a.src_t, sp_off(a, l0 + l, mpos, a.ld_src));
        }
        if (a.sign_out) sg_out = a.sign_out[(uint32_t)mpos % (uint32_t)a.d];
      }
    }
  } else {
    if (u < gb) {
      int gg, k;
      sp_member(a, u, gg, k);
      spos[u] = gg < ng ? (int)sp_pos(a, g0 + gg, k) : -1;
      sslot[u] = sp_lds(a, 0, gg, k);
    }
    __syncthreads();
    const int l = u % LINES;
#pragma unroll
    for (int it = 0; it < LINES; ++it) {
      const int q = u / LINES + kStep * it;
      const int pos = q < gb ? spos[q] : -1;
      if (pos >= 0 && l < nl) v[it] = sp_load(a.src, a.src_t, sp_off(a, l0 + l, pos, a.ld_src));
    }
  }

  // ---- row j of the block of group g (zero beyond b), loaded while the tile
  // is in flight
  const int g = u / a.bp;
  const int j = u - g * a.bp;
  const bool act = j < a.b && g < ng;
  float w[MAXB];
#pragma unroll
  for (int k = 0; k < MAXB; ++k) w[k] = 0.f;
  if (act) {
    if (a.mode == BRQ_HADAMARD) {
#pragma unroll
      for (int k = 0; k < MAXB; ++k)
        if (k < a.b) w[k] = (__popc(j & k) & 1) ? -a.hscale : a.hscale;
    } else {
      const float* row = a.blk + sp_block_row(a, g0 + g, j);
      if (a.blk_vec) {  // rows 16-byte aligned, b a multiple of 4
#pragma unroll
        for (int k4 = 0; k4 < MAXB / 4; ++k4)
          if (4 * k4 < a.b) {
            const float4 q = *reinterpret_cast<const float4*>(row + 4 * k4);
            w[4 * k4] = q.x;
            w[4 * k4 + 1] = q.y;
            w[4 * k4 + 2] = q.z;
            w[4 * k4 + 3] = q.w;
          }
      } else {
#pragma unroll
        for (int k = 0; k < MAXB; ++k)
          if (k < a.b) w[k] = row[k];
      }
    }
  }

  // The optional second stage's block row (pairs run only at radix 16 on the
  // right side, the launcher checks), loaded with the first one so that no
  // global load waits between the two stages.
  const int g2 = u >> 4, j2 = u & 15;
  float w2[16];
  if constexpr (MAXB == 16 && SIDE == 0) {
    if (a.b2) {
      if (a.mode == BRQ_HADAMARD) {
#pragma unroll
        for (int k = 0; k < 16; ++k) w2[k] = (__popc(j2 & k) & 1) ? -0.25f : 0.25f;
      } else {
        const float* row = a.blk2 + sp_block_row2(a, g0, g2, j2);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const float4 q = *reinterpret_cast<const float4*>(row + 4 * k4);
          w2[4 * k4] = q.x;
          w2[4 * k4 + 1] = q.y;
          w2[4 * k4 + 2] = q.z;
          w2[4 * k4 + 3] = q.w;
        }
      }
    }
  }

  // zero the padding members, then write the tile (signs first, forward)
  for (int e = u; e < LINES * a.gw; e += kSpThreads) {
    const int l = e / a.gw, gg = e - l * a.gw;
    for (int k = a.b; k < a.bs; ++k) buf[sp_lds(a, l, gg, k)] = 0.f;
  }
  if (a.side == 0) {
    if (u < gb && mg < ng) {
      const float sg = a.sign_in ? a.sign_in[(uint32_t)mpos % (uint32_t)a.d] : 1.f;
#pragma unroll
      for (int l = 0; l < LINES; ++l)
        if (l < nl) buf[sp_lds(a, l, mg, mk)] = sg * v[l];
    }
  } else {
    const int l = u % LINES;
#pragma unroll
    for (int it = 0; it < LINES; ++it) {
      const int q = u / LINES + kStep * it;
      const int pos = q < gb ? spos[q] : -1;
      if (pos >= 0 && l < nl) {  // left side: one chunk, so the position is the sign index
        const float sg = a.sign_in ? a.sign_in[pos] : 1.f;
        buf[sp_lds(a, l, 0, 0) + sslot[q]] = sg * v[it];
      }
    }
  }
  __syncthreads();

  // ---- y_j = sum_k B[j][k] x_k for every line of the tile, into registers
  float acc[LINES];
  if (act && SIDE == 0) {  // members consecutive: four members per float4
#pragma unroll
    for (int l = 0; l < LINES; ++l) {
      if (l < nl) {
        const float* xr = buf + sp_lds(a, l, g, 0);
        float s = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < MAXB / 4; ++k4) {
          if (4 * k4 < a.bs) {
            const float4 xv = *reinterpret_cast<const float4*>(xr + 4 * k4);
            s = fmaf(w[4 * k4 + 0], xv.x, s);
            s = fmaf(w[4 * k4 + 1], xv.y, s);
            s = fmaf(w[4 * k4 + 2], xv.z, s);
            s = fmaf(w[4 * k4 + 3], xv.w, s);
          }
        }
        acc[l] = s;
      }
    }
  } else if (act) {  // lines consecutive: four lines per float4
#pragma unroll
    for (int l4 = 0; l4 < LINES / 4; ++l4) {
      if (4 * l4 < nl) {
        float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < MAXB; ++k) {
          if (k < a.b) {
            const float4 xv = *reinterpret_cast<const float4*>(buf + sp_lds(a, 4 * l4, g, k));
            s4.x = fmaf(w[k], xv.x, s4.x);
            s4.y = fmaf(w[k], xv.y, s4.y);
            s4.z = fmaf(w[k], xv.z, s4.z);
            s4.w = fmaf(w[k], xv.w, s4.w);
          }
        }
        acc[4 * l4] = s4.x;
        acc[4 * l4 + 1] = s4.y;
        acc[4 * l4 + 2] = s4.z;
        acc[4 * l4 + 3] = s4.w;
      }
    }
  }
  __syncthreads();  // every input read
  if (act) {  // a pair's first stage leaves its outputs in position order
    const bool swap = a.b2 && !a.inv2;
#pragma unroll
    for (int l = 0; l < LINES; ++l)
      if (l < nl) buf[swap ? sp_lds(a, l, j, g) : sp_lds(a, l, g, j)] = acc[l];
  }
  __syncthreads();

  // ---- the optional second stage (radix 16, stride 1) on the same tile: its
  // group g2 is positions 16 g2 .. 16 g2 + 15, consecutive slots (g2, k2)
  if (MAXB == 16 && SIDE == 0 && a.b2) {
    if (a.inv2) {  // members of column g2: slots (k2, g2)
#pragma unroll
      for (int l = 0; l < LINES; ++l) {
        if (l < nl) {
          const float* xr = buf + sp_lds(a, l, 0, g2);
          float s2 = 0.f;
#pragma unroll
          for (int k = 0; k < 16; ++k) s2 = fmaf(w2[k], xr[16 * k], s2);
          acc[l] = s2;
        }
      }
    } else {
#pragma unroll
      for (int l = 0; l < LINES; ++l) {
        if (l < nl) {
          const float* xr = buf + sp_lds(a, l, g2, 0);
          float s2 = 0.f;
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const float4 xv = *reinterpret_cast<const float4*>(xr + 4 * k4);
            s2 = fmaf(w2[4 * k4 + 0], xv.x, s2);
            s2 = fmaf(w2[4 * k4 + 1], xv.y, s2);
            s2 = fmaf(w2[4 * k4 + 2], xv.z, s2);
            s2 = fmaf(w2[4 * k4 + 3], xv.w, s2);
          }
          acc[l] = s2;
        }
      }
    }
    __syncthreads();  // every first-stage output read
#pragma unroll
    for (int l = 0; l < LINES; ++l)
      if (l < nl) buf[sp_lds(a, l, j2, g2)] = acc[l];
    __syncthreads();
  }

  // ---- tile out
  if (a.side == 0) {
    if (u < gb && mg < ng) {
#pragma unroll
      for (int l = 0; l < LINES; ++l)
        if (l < nl)
          sp_store(a.dst, a.dst_t, sp_off(a, l0 + l, mpos, a.ld_dst), sg_out * buf[sp_lds(a, l, mg, mk)]);
    }
  } else {
    const int l = u % LINES;
#pragma unroll
    for (int it = 0; it < LINES; ++it) {
      const int q = u / LINES + kStep * it;
      const int pos = q < gb ? spos[q] : -1;
      if (pos >= 0 && l < nl) {
        const float sg = a.sign_out ? a.sign_out[pos] : 1.f;
        sp_store(a.dst, a.dst_t, sp_off(a, l0 + l, pos, a.ld_dst), sg * buf[sp_lds(a, l, 0, 0) + sslot[q]]);
      }
    }
  }
}

template <int MAXB>
hipError_t launch_t(const SpArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)sp_blocks(a));
  if (a.side)
    hipLaunchKernelGGL((stage_kernel<MAXB, 1, kSpLines>), grid, dim3(kSpThreads), 0, s, a);
  else if (sp_tl(a) == kSpLinesTiny)
    hipLaunchKernelGGL((stage_kernel<MAXB, 0, kSpLinesTiny>), grid, dim3(kSpThreads), 0, s, a);
  else if (sp_tl(a) == kSpLinesFew)
    hipLaunchKernelGGL((stage_kernel<MAXB, 0, kSpLinesFew>), grid, dim3(kSpThreads), 0, s, a);
  else
    hipLaunchKernelGGL((stage_kernel<MAXB, 0, kSpLines>), grid, dim3(kSpThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stage(const SpArgs& a, hipStream_t s) {
  if (a.b2 && (a.bp != 16 || a.side != 0)) return hipErrorInvalidValue;  // pairs: radix 16, right side
  if (a.bp <= 8) return launch_t<8>(a, s);
  if (a.bp <= 16) return launch_t<16>(a, s);
  if (a.bp <= 32) return launch_t<32>(a, s);
  return launch_t<64>(a, s);
}

}  // namespace brq
