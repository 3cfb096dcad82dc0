// Generic tile pass: one workgroup loads a 2-D tile of the matrix into LDS as
// float32, applies the stages of this pass along either axis (left-side stages
// mix rows, right-side stages mix columns), and stores the tile or quantizes
// and packs it.  Every plan shape goes through here; the fused MFMA kernels
// cover the common shapes faster.
//
// Stage arithmetic ([HARP] technical summary 2.1): for each group c of stage t,
// y[base + j*S_t] = sum_k B_{t,c}[j][k] x[base + k*S_t], the group index being
// c = (i / (b_t*S_t))*S_t + i % S_t for any member i.  Hadamard blocks are
// H_b/sqrt(b) with H_b[j][k] = (-1)^popcount(j & k) (natural Sylvester order).
#include "brq_internal.h"

namespace brq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float load_elem(const void* p, int t, int64_t i) {
  if (t == BRQ_F32) return static_cast<const float*>(p)[i];
  if (t == BRQ_BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  return (float)static_cast<const _Float16*>(p)[i];
}

__device__ __forceinline__ void store_elem(void* p, int t, int64_t i, float v) {
  if (t == BRQ_F32) static_cast<float*>(p)[i] = v;
  else if (t == BRQ_BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else static_cast<_Float16*>(p)[i] = (_Float16)v;
}

// Apply one stage along axis `axis` of the LDS tile.  Each thread owns whole
// groups of one line, so the update is in place without a barrier inside.
template <int MAXB>
__device__ void stage_apply(float* lds, int ldl, int axis, const StageDesc& st,
                            const AxisDesc& ax, int64_t relbase, int nlines) {
  const int b = st.b;
  const int ngroups = (ax.P / b) * ax.W;
  const int units = ngroups * nlines;
  const float rs = (st.mode == BRQ_HADAMARD) ? rsqrtf((float)b) : 1.0f;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int gid = u / nlines;
    const int line = u - gid * nlines;
    const TileGroup tg = tile_group(st, ax, gid);
    const int a0 = axis ? (line * ldl + tg.e0) : (tg.e0 * ldl + line);
    const int astep = axis ? tg.estep : tg.estep * ldl;
    float xs[MAXB];
#pragma unroll
    for (int j = 0; j < MAXB; ++j)
      if (j < b) xs[j] = lds[a0 + j * astep];
    if (st.mode == BRQ_HADAMARD) {
      for (int jo = 0; jo < b; ++jo) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < MAXB; ++k)
          if (k < b) acc += (__popc(jo & k) & 1) ? -xs[k] : xs[k];
        lds[a0 + jo * astep] = acc * rs;
      }
    } else {
      const float* blk = st.blk;
      if (st.mode == BRQ_PER_GROUP) blk += group_index(st, ax, relbase, tg) * b * b;
      for (int jo = 0; jo < b; ++jo) {
        const float* row = blk + jo * b;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < MAXB; ++k)
          if (k < b) acc = fmaf(row[k], xs[k], acc);
        lds[a0 + jo * astep] = acc;
      }
    }
  }
}

__device__ void apply_stage(float* lds, int ldl, int axis, const StageDesc& st,
                            const AxisDesc& ax, int64_t relbase, int nlines) {
  if (st.b <= 4) stage_apply<4>(lds, ldl, axis, st, ax, relbase, nlines);
  else if (st.b <= 8) stage_apply<8>(lds, ldl, axis, st, ax, relbase, nlines);
  else if (st.b <= 16) stage_apply<16>(lds, ldl, axis, st, ax, relbase, nlines);
  else if (st.b <= 32) stage_apply<32>(lds, ldl, axis, st, ax, relbase, nlines);
  else stage_apply<64>(lds, ldl, axis, st, ax, relbase, nlines);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void pass_kernel(PassArgs a) {
  extern __shared__ float lds[];
  const AxisDesc& X0 = a.ax[0];
  const AxisDesc& X1 = a.ax[1];
  const int64_t tiles_c = axis_tiles(X1);
  const int64_t tid_r = (int64_t)blockIdx.x / tiles_c;
  const int64_t tid_c = (int64_t)blockIdx.x - tid_r * tiles_c;
  const AxisPos pr = axis_pos(X0, tid_r);
  const AxisPos pc = axis_pos(X1, tid_c);
  const int RT = X0.P * X0.W;
  const int CT = X1.P * X1.W;
  const int ldl = CT + 1;
  const int nel = RT * CT;

  // ---- prologue: load (or unpack + dequantize) into LDS as float32
  for (int e = threadIdx.x; e < nel; e += blockDim.x) {
    const int er = e / CT;
    const int ec = e - er * CT;
    float v = 0.f;
    if (er < pr.limit && ec < pc.limit) {
      const int64_t row = pr.base + axis_off(X0, er);
      const int64_t col = pc.base + axis_off(X1, ec);
      if (a.pro == PRO_LOAD) {
        v = load_elem(a.src, a.src_t, row * a.ld_src + col);
      } else {
        const int64_t bit = col * a.bits;
        const uint8_t* crow = a.in_codes + row * a.codes_ld;
        const int64_t byte = bit >> 3;
        uint32_t win = crow[byte];
        if (byte + 1 < a.codes_ld) win |= (uint32_t)crow[byte + 1] << 8;
        const int code = (int)((win >> (bit & 7)) & ((1u << a.bits) - 1u));
        const int64_t sidx = row * a.scales_ld + col / a.group;
        if (a.qkind == BRQ_ABSMAX) {
          const float alpha = static_cast<const float*>(a.in_scales)[sidx];
          v = alpha * ((float)code / a.h - 1.0f);
        } else {
          const float r = (float)static_cast<const _Float16*>(a.in_scales)[sidx];
          v = r * a.cent[code] / a.sqrt_g;
        }
      }
      if (!a.inverse) {
        if (X0.sign) v *= X0.sign[row % X0.sign_mod];
        if (X1.sign) v *= X1.sign[col % X1.sign_mod];
      }
    }
    lds[er * ldl + ec] = v;
  }
  __syncthreads();

  // ---- stages (the two sides commute, so axis order within a pass is free)
  for (int s = 0; s < X0.nst; ++s) {
    apply_stage(lds, ldl, 0, X0.st[s], X0, pr.relbase, CT);
    __syncthreads();
  }
  for (int s = 0; s < X1.nst; ++s) {
    apply_stage(lds, ldl, 1, X1.st[s], X1, pc.relbase, RT);
    __syncthreads();
  }

  // ---- epilogue
  if (a.epi == EPI_STORE) {
    for (int e = threadIdx.x; e < nel; e += blockDim.x) {
      const int er = e / CT;
      const int ec = e - er * CT;
      if (er < pr.limit && ec < pc.limit) {
        const int64_t row = pr.base + axis_off(X0, er);
        const int64_t col = pc.base + axis_off(X1, ec);
        float v = lds[er * ldl + ec];
        if (a.inverse) {
          if (X0.sign) v *= X0.sign[row % X0.sign_mod];
          if (X1.sign) v *= X1.sign[col % X1.sign_mod];
        }
        store_elem(a.dst, a.dst_t, row * a.ld_dst + col, v);
      }
    }
    return;
  }

  // Quantize: the tile's columns are contiguous and hold whole groups.
  // One wave per (row, group); a uniform round count keeps barriers legal.
  __shared__ uint8_t cs[kThreads / 64][1024];
  const int g = a.group;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int gpr = CT / g;
  const int units = RT * gpr;
  const int lv = a.nlev - 1;
  for (int r0 = 0; r0 < units; r0 += nwaves) {
    const int u = r0 + wave;
    const int er = u / gpr;
    const int gi = u - er * gpr;
    const bool active = (u < units) && (er < pr.limit) && ((int64_t)gi * g < pc.limit);
    if (active) {
      const float* v = lds + er * ldl + gi * g;
      float stat = 0.f;
      if (a.qkind == BRQ_ABSMAX) {
        for (int t = lane; t < g; t += 64) stat = fmaxf(stat, fabsf(v[t]));
        stat = wave_max(stat);
        const float k = stat > 0.f ? a.h / stat : 0.f;
        for (int t = lane; t < g; t += 64) {
          int c = 0;
          if (stat > 0.f) {
            c = (int)rintf(fmaf(v[t], k, a.h));
            c = c < 0 ? 0 : (c > lv ? lv : c);
          }
          cs[wave][t] = (uint8_t)c;
        }
      } else {
        for (int t = lane; t < g; t += 64) stat = fmaf(v[t], v[t], stat);
        stat = sqrtf(wave_sum(stat));
        const float k = stat > 0.f ? a.sqrt_g / stat : 0.f;
        for (int t = lane; t < g; t += 64) {
          int c = 0;
          if (stat > 0.f) {
            const float z = v[t] * k;
            for (int q = 0; q < lv; ++q) c += (z > a.tau[q]) ? 1 : 0;
          }
          cs[wave][t] = (uint8_t)c;
        }
      }
      const int64_t row = pr.base + er;
      const int64_t gcol = (pc.base + (int64_t)gi * g) / g;
      if (lane == 0) {
        if (a.qkind == BRQ_ABSMAX)
          static_cast<float*>(a.scales)[row * a.scales_ld + gcol] = stat;
        else
          static_cast<_Float16*>(a.scales)[row * a.scales_ld + gcol] = (_Float16)stat;
      }
    }
    __syncthreads();
    if (active) {
      const int64_t row = pr.base + er;
      const int64_t gcol = (pc.base + (int64_t)gi * g) / g;
      const int nbytes = g * a.bits / 8;
      uint8_t* out = a.codes + row * a.codes_ld + gcol * nbytes;
      for (int p = lane; p < nbytes; p += 64) {
        const int e0 = (8 * p) / a.bits;
        int e1 = (8 * p + 7) / a.bits;
        if (e1 >= g) e1 = g - 1;
        uint32_t byte = 0;
        for (int e = e0; e <= e1; ++e) {
          const int sh = e * a.bits - 8 * p;
          const uint32_t c = cs[wave][e];
          byte |= sh >= 0 ? (c << sh) : (c >> (-sh));
        }
        out[p] = (uint8_t)(byte & 0xffu);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_pass(const PassArgs& a, hipStream_t s) {
  const int64_t tiles = axis_tiles(a.ax[0]) * axis_tiles(a.ax[1]);
  if (tiles <= 0) return hipSuccess;
  const int RT = a.ax[0].P * a.ax[0].W;
  const int CT = a.ax[1].P * a.ax[1].W;
  const size_t lds = (size_t)RT * (CT + 1) * sizeof(float);
  static bool attr_set = false;  // LDS above 64 KiB needs the opt-in attribute
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pass_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (lds > 96 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pass_kernel, dim3((unsigned)tiles), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace brq
