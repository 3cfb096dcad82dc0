// Right-side stages of radix <= 8 with one group per lane (stage.h).
#include "stage.h"

namespace brq {
namespace {

// Element types: float, bfloat16 (as its bits) and half.
struct Bf16 {};
template <typename T> struct Elem;
template <> struct Elem<float> {
  using S = float;
  static __device__ __forceinline__ float in(S v) { return v; }
  static __device__ __forceinline__ S out(float v) { return v; }
};
template <> struct Elem<Bf16> {
  using S = uint16_t;
  static __device__ __forceinline__ float in(S v) { return __uint_as_float((uint32_t)v << 16); }
  static __device__ __forceinline__ S out(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) u |= 0x400000u;  // keep NaN a quiet NaN
    else u += 0x7fffu + ((u >> 16) & 1u);                   // nearest, ties to even
    return (uint16_t)(u >> 16);
  }
};
template <> struct Elem<_Float16> {
  using S = _Float16;
  static __device__ __forceinline__ float in(S v) { return (float)v; }
  static __device__ __forceinline__ S out(float v) { return (_Float16)v; }
};

template <int B> constexpr int sl_pitch() { return B * B + 1; }  // odd: no bank conflicts

template <int B, typename TI, typename TO>
__device__ __forceinline__ void sl_body(const SpArgs& a, int rows_per, float* blds) {
  constexpr int BB = B * B, P = sl_pitch<B>();
  using SI = typename Elem<TI>::S;
  using SO = typename Elem<TO>::S;
  const SI* src = static_cast<const SI*>(a.src);
  SO* dst = static_cast<SO*>(a.dst);
  const int l = threadIdx.x & (kSlLanes - 1), w = threadIdx.x / kSlLanes;
  const uint32_t lo_tiles = (uint32_t)(a.ngroups / kSlLanes);
  const uint32_t t = blockIdx.x % lo_tiles, rt = blockIdx.x / lo_tiles;
  const int64_t gid = sl_group(t, l);

  // the 64 groups' blocks are contiguous (per group) or one shared block
  if (a.mode != BRQ_HADAMARD) {
    const int64_t base = a.mode == BRQ_PER_GROUP ? sp_block_row(a, sl_group(t, 0), 0) : 0;
    const int n = a.mode == BRQ_PER_GROUP ? kSlLanes * BB : BB;
    for (int e = threadIdx.x; e < kSlLanes * BB; e += kSlThreads) {
      const int g = e / BB, r = e - g * BB;
      blds[g * P + r] = a.blk[base + (e < n ? e : r)];
    }
    __syncthreads();
  }
  // member k sits at pos0 + k S; the signs fold into the block (exact:
  // +-1 scalings), diag(sign_out) B diag(sign_in)
  const int64_t pos0 = sp_pos(a, gid, 0);
  const int64_t S = a.S;
  const uint32_t ip0 = (uint32_t)pos0 % (uint32_t)a.d;
  float wm[B][B];
#pragma unroll
  for (int j = 0; j < B; ++j)
#pragma unroll
    for (int k = 0; k < B; ++k) {
      float v = a.mode == BRQ_HADAMARD ? ((__popc(j & k) & 1) ? -a.hscale : a.hscale)
                                       : blds[l * P + j * B + k];
      if (a.sign_in) v *= a.sign_in[ip0 + (uint32_t)(k * S)];
      if (a.sign_out) v *= a.sign_out[ip0 + (uint32_t)(j * S)];
      wm[j][k] = v;
    }

  // rows rt * rows_per + w + 4 i, two at a time
  const int64_t r0 = (int64_t)rt * rows_per + w;
  const int64_t rend = r0 - w + rows_per < a.lines ? r0 - w + rows_per : a.lines;
  for (int64_t r = r0; r < rend; r += 8) {
    const bool two = r + 4 < rend;
    const SI* s0 = src + r * a.ld_src;
    const SI* s1 = src + (two ? r + 4 : r) * a.ld_src;
    float x0[B], x1[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      x0[k] = Elem<TI>::in(s0[pos0 + k * S]);
      x1[k] = Elem<TI>::in(s1[pos0 + k * S]);
    }
    SO* d0 = dst + r * a.ld_dst;
    SO* d1 = dst + (r + 4) * a.ld_dst;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        y0 = fmaf(wm[j][k], x0[k], y0);
        y1 = fmaf(wm[j][k], x1[k], y1);
      }
      d0[pos0 + j * S] = Elem<TO>::out(y0);
      if (two) d1[pos0 + j * S] = Elem<TO>::out(y1);
    }
  }
}

// Radix 16: a block is 256 floats, so wave w keeps rows 4w .. 4w + 3 of its
// lane's block (64 floats) and makes those four outputs for every row of the
// workgroup's range; the four waves read the same inputs (from cache after
// the first).  In place, a wave's outputs are other waves' inputs, so the
// waves meet at a barrier between the reads and the writes of each row pair.
template <typename TI, typename TO>
__device__ __forceinline__ void sl_body16(const SpArgs& a, int rows_per) {
  constexpr int B = 16, JW = 4;
  using SI = typename Elem<TI>::S;
  using SO = typename Elem<TO>::S;
  const SI* src = static_cast<const SI*>(a.src);
  SO* dst = static_cast<SO*>(a.dst);
  const int l = threadIdx.x & (kSlLanes - 1), w = threadIdx.x / kSlLanes;
  const uint32_t lo_tiles = (uint32_t)(a.ngroups / kSlLanes);
  const uint32_t t = blockIdx.x % lo_tiles, rt = blockIdx.x / lo_tiles;
  const int64_t gid = sl_group(t, l);
  const int64_t pos0 = sp_pos(a, gid, 0);
  const int64_t S = a.S;
  const uint32_t ip0 = (uint32_t)pos0 % (uint32_t)a.d;
  float wq[JW][B];
  if (a.mode == BRQ_HADAMARD) {
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int k = 0; k < B; ++k) wq[jj][k] = (__popc((JW * w + jj) & k) & 1) ? -a.hscale : a.hscale;
  } else {
    const float* row = a.blk + sp_block_row(a, gid, JW * w);
#pragma unroll
    for (int q = 0; q < JW * B / 4; ++q) {  // 16-byte aligned: the host checks blk_vec
      const float4 v = *reinterpret_cast<const float4*>(row + 4 * q);
      wq[q / 4][4 * (q % 4)] = v.x;
      wq[q / 4][4 * (q % 4) + 1] = v.y;
      wq[q / 4][4 * (q % 4) + 2] = v.z;
      wq[q / 4][4 * (q % 4) + 3] = v.w;
    }
  }
#pragma unroll
  for (int jj = 0; jj < JW; ++jj)
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (a.sign_in) wq[jj][k] *= a.sign_in[ip0 + (uint32_t)(k * S)];
      if (a.sign_out) wq[jj][k] *= a.sign_out[ip0 + (uint32_t)((JW * w + jj) * S)];
    }
  const bool in_place = a.src == a.dst;
  const int64_t rb = (int64_t)rt * rows_per;
  const int64_t rend = rb + rows_per < a.lines ? rb + rows_per : a.lines;
  for (int64_t r = rb; r < rend; r += 2) {  // the same trip count for every wave
    const bool two = r + 1 < rend;
    const SI* s0 = src + r * a.ld_src;
    const SI* s1 = src + (two ? r + 1 : r) * a.ld_src;
    float x0[B], x1[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      x0[k] = Elem<TI>::in(s0[pos0 + k * S]);
      x1[k] = Elem<TI>::in(s1[pos0 + k * S]);
    }
    if (in_place) __syncthreads();  // every wave has read both rows
    SO* d0 = dst + r * a.ld_dst;
    SO* d1 = dst + (r + 1) * a.ld_dst;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        y0 = fmaf(wq[jj][k], x0[k], y0);
        y1 = fmaf(wq[jj][k], x1[k], y1);
      }
      d0[pos0 + (JW * w + jj) * S] = Elem<TO>::out(y0);
      if (two) d1[pos0 + (JW * w + jj) * S] = Elem<TO>::out(y1);
    }
  }
}

template <typename TI>
__device__ __forceinline__ void sl_out16(const SpArgs& a, int rows_per) {
  if (a.dst_t == BRQ_F32) sl_body16<TI, float>(a, rows_per);
  else if (a.dst_t == BRQ_BF16) sl_body16<TI, Bf16>(a, rows_per);
  else sl_body16<TI, _Float16>(a, rows_per);
}

__global__ __launch_bounds__(kSlThreads) void stage_lanes16_kernel(SpArgs a, int rows_per) {
  if (a.src_t == BRQ_F32) sl_out16<float>(a, rows_per);
  else if (a.src_t == BRQ_BF16) sl_out16<Bf16>(a, rows_per);
  else sl_out16<_Float16>(a, rows_per);
}

template <int B, typename TI>
__device__ __forceinline__ void sl_out(const SpArgs& a, int rows_per, float* blds) {
  if (a.dst_t == BRQ_F32) sl_body<B, TI, float>(a, rows_per, blds);
  else if (a.dst_t == BRQ_BF16) sl_body<B, TI, Bf16>(a, rows_per, blds);
  else sl_body<B, TI, _Float16>(a, rows_per, blds);
}

template <int B>
__global__ __launch_bounds__(kSlThreads) void stage_lanes_kernel(SpArgs a, int rows_per) {
  __shared__ float blds[kSlLanes * sl_pitch<B>()];
  if (a.src_t == BRQ_F32) sl_out<B, float>(a, rows_per, blds);
  else if (a.src_t == BRQ_BF16) sl_out<B, Bf16>(a, rows_per, blds);
  else sl_out<B, _Float16>(a, rows_per, blds);
}

template <int B>
hipError_t launch_t(const SpArgs& a, int rows_per, hipStream_t s) {
  const SlGeom g = sl_geom(a, rows_per);
  hipLaunchKernelGGL(stage_lanes_kernel<B>, dim3((unsigned)(g.lo_tiles * g.row_tiles)),
                     dim3(kSlThreads), 0, s, a, rows_per);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stage_lanes(const SpArgs& a, int rows_per, hipStream_t s) {
  switch (a.b) {
    case 2: return launch_t<2>(a, rows_per, s);
    case 3: return launch_t<3>(a, rows_per, s);
    case 4: return launch_t<4>(a, rows_per, s);
    case 5: return launch_t<5>(a, rows_per, s);
    case 6: return launch_t<6>(a, rows_per, s);
    case 7: return launch_t<7>(a, rows_per, s);
    case 8: return launch_t<8>(a, rows_per, s);
    case 16: {
      const SlGeom g = sl_geom(a, rows_per);
      hipLaunchKernelGGL(stage_lanes16_kernel, dim3((unsigned)(g.lo_tiles * g.row_tiles)),
                         dim3(kSlThreads), 0, s, a, rows_per);
      return hipGetLastError();
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace brq
