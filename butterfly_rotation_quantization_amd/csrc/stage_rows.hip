// Left-side stages by whole rows (stage.h): one group and a run of columns
// per workgroup, inputs in registers, block entries through the scalar cache.
#include "stage.h"

namespace brq {
namespace {

// VEC consecutive elements of one row as float32.
template <typename T, int VEC>
struct RowIO;

template <int VEC>
struct RowIO<float, VEC> {
  static __device__ __forceinline__ void load(const void* p, int64_t i, float (&o)[VEC]) {
    const float* q = static_cast<const float*>(p) + i;
    if constexpr (VEC == 4) {
      const float4 v = *reinterpret_cast<const float4*>(q);
      o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (VEC == 2) {
      const float2 v = *reinterpret_cast<const float2*>(q);
      o[0] = v.x; o[1] = v.y;
    } else {
      o[0] = q[0];
    }
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, const float (&v)[VEC]) {
    float* q = static_cast<float*>(p) + i;
    if constexpr (VEC == 4) {
      *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (VEC == 2) {
      *reinterpret_cast<float2*>(q) = make_float2(v[0], v[1]);
    } else {
      q[0] = v[0];
    }
  }
};

// 16-bit types: the VEC halves travel as one 2 VEC-byte word.
__device__ __forceinline__ float bf16_to_f(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t f_to_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) u |= 0x400000u;  // keep NaN a quiet NaN
  else u += 0x7fffu + ((u >> 16) & 1u);                   // nearest, ties to even
  return u >> 16;
}
__device__ __forceinline__ float f16_to_f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f_to_f16(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

template <bool BF, int VEC>
struct Row16 {
  static __device__ __forceinline__ float cvt(uint32_t h) { return BF ? bf16_to_f(h) : f16_to_f(h); }
  static __device__ __forceinline__ uint32_t back(float v) { return BF ? f_to_bf16(v) : f_to_f16(v); }
  static __device__ __forceinline__ void load(const void* p, int64_t i, float (&o)[VEC]) {
    const uint16_t* q = static_cast<const uint16_t*>(p) + i;
    if constexpr (VEC == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(q);
      o[0] = cvt(v.x & 0xffffu); o[1] = cvt(v.x >> 16); o[2] = cvt(v.y & 0xffffu); o[3] = cvt(v.y >> 16);
    } else if constexpr (VEC == 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(q);
      o[0] = cvt(v & 0xffffu); o[1] = cvt(v >> 16);
    } else {
      o[0] = cvt(q[0]);
    }
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, const float (&v)[VEC]) {
    uint16_t* q = static_cast<uint16_t*>(p) + i;
    if constexpr (VEC == 4) {
      *reinterpret_cast<uint2*>(q) = make_uint2(back(v[0]) | back(v[1]) << 16, back(v[2]) | back(v[3]) << 16);
    } else if constexpr (VEC == 2) {
      *reinterpret_cast<uint32_t*>(q) = back(v[0]) | back(v[1]) << 16;
    } else {
      q[0] = (uint16_t)back(v[0]);
    }
  }
};
template <int VEC> struct RowIO<__bf16, VEC> : Row16<true, VEC> {};
template <int VEC> struct RowIO<_Float16, VEC> : Row16<false, VEC> {};

// The block and sign tables as constant memory: the kernel never writes
// them, and uniform loads from the constant address space become scalar
// loads (a generic pointer could alias the output, which forces vector loads).
typedef const __attribute__((address_space(4))) float* cfloat_p;
__device__ __forceinline__ cfloat_p as_const(const float* p) { return (cfloat_p)(uintptr_t)p; }

template <int B, int VEC, bool HAD, typename TI, typename TO>
__device__ __forceinline__ void sr_body(const SpArgs& a) {
  const uint32_t nct = (uint32_t)sr_col_tiles(a);
  uint32_t gid, ct;
  sr_tile_of_block(blockIdx.x, nct, gid, ct);
  const int64_t c0 = sr_col(ct, threadIdx.x, VEC);
  if (c0 >= a.lines) return;  // the host keeps lines a multiple of VEC

  // the group's B rows (positions along the transformed axis = matrix rows)
  float x[B][VEC];
#pragma unroll
  for (int k = 0; k < B; ++k) {
    RowIO<TI, VEC>::load(a.src, sp_pos(a, gid, k) * a.ld_src + c0, x[k]);
  }
  if (a.sign_in) {
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const float sg = as_const(a.sign_in)[sp_pos(a, gid, k)];
#pragma unroll
      for (int v = 0; v < VEC; ++v) x[k][v] *= sg;
    }
  }

  // the block is the same for every thread of the workgroup, so its entries
  // are scalar loads
  const cfloat_p blk = HAD ? nullptr : as_const(a.blk) + sp_block_row(a, gid, 0);
  // wide blocks: a few rows per iteration keep the block entries held in
  // scalar registers few
#pragma unroll(B <= 16 ? B : 2)
  for (int j = 0; j < B; ++j) {
    float y[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) y[v] = 0.f;
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const float w = HAD ? ((__builtin_popcount(j & k) & 1) ? -a.hscale : a.hscale) : blk[j * B + k];
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[v] = fmaf(w, x[k][v], y[v]);
    }
    const int64_t row = sp_pos(a, gid, j);
    if (a.sign_out) {
      const float sg = as_const(a.sign_out)[row];
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[v] *= sg;
    }
    RowIO<TO, VEC>::store(a.dst, row * a.ld_dst + c0, y);
  }
}

// Type pairs: float32 in or out (a plan's first stage reads the caller's
// type into the float32 intermediate, its last writes the caller's type).
template <int B, bool HAD>
__global__ __launch_bounds__(kSrThreads) void stage_rows_kernel(SpArgs a) {
  constexpr int VEC = sr_vec(B);
  if (a.src_t == BRQ_F32) {
    if (a.dst_t == BRQ_F32) sr_body<B, VEC, HAD, float, float>(a);
    else if (a.dst_t == BRQ_BF16) sr_body<B, VEC, HAD, float, __bf16>(a);
    else sr_body<B, VEC, HAD, float, _Float16>(a);
  } else if (a.src_t == BRQ_BF16) {
    sr_body<B, VEC, HAD, __bf16, float>(a);
  } else {
    sr_body<B, VEC, HAD, _Float16, float>(a);
  }
}

template <int B>
hipError_t launch_t(const SpArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(sr_col_tiles(a) * a.ngroups));
  if constexpr (B <= 16) {
    if (a.mode == BRQ_HADAMARD) {
      hipLaunchKernelGGL((stage_rows_kernel<B, true>), grid, dim3(kSrThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((stage_rows_kernel<B, false>), grid, dim3(kSrThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stage_rows(const SpArgs& a, hipStream_t s) {
  switch (a.b) {
    case 2: return launch_t<2>(a, s);
    case 4: return launch_t<4>(a, s);
    case 8: return launch_t<8>(a, s);
    case 16: return launch_t<16>(a, s);
    case 32: return launch_t<32>(a, s);
    case 64: return launch_t<64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace brq
