// Fast path for two-sided plans of the shape U = (bU, 16, 16), V = (bV, 16, 16)
// (bU = 16, bV <= 64): two kernels on MFMA 16x16x4 float32 tiles.
//
//  pass A: the stride-256 stages U_0 and V_0.  Rows r0*256 + q (r0 < 16) and
//          columns c0*256 + p (c0 < bV) of one (q, p) pair form a 16 x bV
//          matrix X_qp; the pass computes B^U0_q X_qp (B^V0_p)^T for every
//          (q, p) and writes the float32 intermediate.
//  pass B: the remaining radix-16 stages U_1, U_2, V_1, V_2 on a 256 x 256
//          block (rows r0*256 + [0,256), columns c0*256 + [0,256)) held in
//          registers, with one LDS exchange, then the group quantizer and
//          LSB-first packing.
//
// The index arithmetic both kernels use lives here as __host__ __device__
// functions so the host dry run checks exactly what the GPU executes.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kFaWaves = 8;            // pass A: waves per workgroup (one p each)
constexpr int kFaP = kFaWaves;         // pass A: p values per workgroup
constexpr int kFaQC = 16;              // pass A: q values per workgroup (looped)
constexpr int kFbWaves = 16;           // pass B: waves per workgroup
// pass B LDS: the exchange buffer [r1 16][c1h 8][r2 16][c2 16] (swizzled),
// whose first 16 KB hold the tile's 16 V_1 blocks during phase 1, then the
// tile's 16 V_2 blocks.
constexpr int kFbXchFloats = 16 * 8 * 16 * 16;
constexpr int kFbV1Off = 0;
constexpr int kFbV2Off = kFbXchFloats;
constexpr int kFbLdsFloats = kFbV2Off + 16 * 256;

struct FusedAArgs {
  const void* w;      // input [m][n], type wt, leading dimension ldw
  int wt;
  int64_t ldw;
  float* ws;          // float32 intermediate [m][n], leading dimension n
  int64_t m, n;
  int bv;             // radix of V_0 (columns)
  int nb;             // 16-blocks spanned by bv (padded K = N = 16*nb)
  int nchunk;         // n / d_V (block-diagonal right side)
  int dv;             // d_V = bv * 256
  const float* u0;    // U_0 blocks [256][16][16] (or one shared block), signs folded in
  int64_t u0_gs;      // float stride between groups (0 = shared)
  const float* v0;    // V_0 blocks padded [256][16nb][16nb] (or one), signs folded in
  int64_t v0_gs;
  int nqc;            // q chunks: 256 / kFaQC
  uint32_t bv_magic;  // floor(2^32 / bv) + 1: i / bv = (i * bv_magic) >> 32 for the i used
  int64_t u0_n, v0_n; // float extents of the block arrays (host checks)
};

struct FusedBArgs {
  const float* ws;    // float32 intermediate from pass A
  int64_t m, n;
  int bv;             // radix of V_0: column chunks c0 per d_V
  int nchunk, dv;
  const float* u1; int64_t u1_gs;  // U_1 blocks [256][16][16], group r0*16 + r2
  const float* u2; int64_t u2_gs;  // U_2 blocks, group r0*16 + r1
  const float* v1; int64_t v1_gs;  // V_1 blocks, group c0*16 + c2
  const float* v2; int64_t v2_gs;  // V_2 blocks, group c0*16 + c1
  // quantizer
  int qkind, bits, group, nlev;
  float h, sqrt_g;
  float tau[kMaxLevels];
  uint8_t* codes;
  void* scales;
  int64_t codes_ld, scales_ld;
  int64_t u1_n, u2_n, v1_n, v2_n;  // float extents of the block arrays (host checks)
};

// ---- pass A geometry --------------------------------------------------------

// Workgroup b -> (p range, q chunk, column chunk).  Workgroups are dealt to
// the 8 XCDs round robin (b % 8); consecutive slots of one XCD walk the p
// ranges first, so workgroups sharing input rows share that XCD's L2.
struct FaTile {
  int p0, q0, chunk;
};

__host__ __device__ inline FaTile fa_tile(const FusedAArgs& a, int64_t b, int64_t nwg) {
  const int64_t per_xcd = nwg / 8;
  const int64_t lin = (b % 8) * per_xcd + b / 8;
  FaTile t;
  t.p0 = (int)(lin % (256 / kFaP)) * kFaP;
  const int64_t rest = lin / (256 / kFaP);
  t.q0 = (int)(rest % a.nqc) * kFaQC;
  t.chunk = (int)(rest / a.nqc);
  return t;
}

__host__ __device__ inline int64_t fa_nwg(const FusedAArgs& a) {
  return (int64_t)(256 / kFaP) * a.nqc * a.nchunk;
}

// i / bv without a division instruction (exact for the ranges the host checks).
__host__ __device__ inline int fa_div_bv(const FusedAArgs& a, int i) {
  return (int)(((uint64_t)(uint32_t)i * a.bv_magic) >> 32);
}

// LDS input slot of (p_local, r0, c0): [p kFaP][r0 16][16*nb + 4]
__host__ __device__ inline int fa_kp(int nb) { return 16 * nb + 4; }
__host__ __device__ inline int fa_lds_in(int nb, int pl, int r0, int c0) {
  return (pl * 16 + r0) * fa_kp(nb) + c0;
}
// LDS output slot of (r0, c0, p_local): [r0 16][c0 bv][p kFaP + 4].  The pad
// spreads the accumulator writes (lanes over r0 and c0) over more banks and
// keeps each p run 16-byte aligned for the float4 reads of the store.
constexpr int kFaOutStride = kFaP + 4;
__host__ __device__ inline int fa_lds_out(int bv, int r0, int c0, int pl) {
  return (r0 * bv + c0) * kFaOutStride + pl;
}
__host__ __device__ inline int fa_lds_floats(int nb, int bv) {
  const int in = kFaP * 16 * fa_kp(nb);
  const int out = 16 * bv * kFaOutStride;
  return in > out ? in : out;
}
// Global element (row, col) of (r0, q) x (chunk, c0, p).
__host__ __device__ inline int64_t fa_row(int r0, int q) { return (int64_t)r0 * 256 + q; }
__host__ __device__ inline int64_t fa_col(const FusedAArgs& a, int chunk, int c0, int p) {
  return (int64_t)chunk * a.dv + (int64_t)c0 * 256 + p;
}

// ---- pass B geometry --------------------------------------------------------

struct FbTile {
  int r0, c0, chunk;
};

__host__ __device__ inline int64_t fb_nwg(const FusedBArgs& a) {
  return (int64_t)16 * a.bv * a.nchunk;
}

__host__ __device__ inline FbTile fb_tile(const FusedBArgs& a, int64_t b) {
  FbTile t;
  t.r0 = (int)(b % 16);
  const int64_t rest = b / 16;
  t.c0 = (int)(rest % a.bv);
  t.chunk = (int)(rest / a.bv);
  return t;
}

// Exchange slot of element (r1, c1h, r2, c2).  The XOR swizzles keep the
// float4 reads of phase 2 (4 consecutive c2) contiguous while spreading the
// scalar writes of phase 1 (lanes over r1 and c1h) over 8 banks instead of 1.
__host__ __device__ inline int fb_xch(int r1, int c1h, int r2, int c2) {
  return ((r1 * 8 + c1h) * 16 + (r2 ^ (c1h >> 2))) * 16 + (c2 ^ ((r1 & 3) << 2));
}

__host__ __device__ inline int64_t fb_row(const FbTile& t, int r1, int r2) {
  return (int64_t)t.r0 * 256 + r1 * 16 + r2;
}
__host__ __device__ inline int64_t fb_col(const FusedBArgs& a, const FbTile& t, int c1, int c2) {
  return (int64_t)t.chunk * a.dv + (int64_t)t.c0 * 256 + c1 * 16 + c2;
}

// ---- entry points -------------------------------------------------------------

hipError_t fused_prepare(Plan& p, const float* host_blocks, const int8_t* host_signs);
void fused_release(Plan& p);

bool fused_rotate_supported(const Plan* U, const Plan* V, int xt, int yt, int64_t rows,
                            int64_t cols, int64_t ldx, int64_t ldy, const void* x, const void* y);
hipError_t fused_rotate(const Plan* U, const Plan* V, const void* x, int xt, int64_t ldx, void* y,
                        int yt, int64_t ldy, int64_t rows, int64_t cols, hipStream_t s);

bool fused_rqp_supported(const Plan* U, const Plan* V, int wt, int64_t m, int64_t n, int64_t ldw,
                         const void* w, const brq_quant* q);
brq_status fused_rqp(const Plan* U, const Plan* V, const void* w, int wt, int64_t m, int64_t n,
                     int64_t ldw, const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                     size_t ws_bytes, hipStream_t s);

// Kernel launchers (fused_kernels.hip; the dry-run build walks their indices).
// Pass B is persistent: `grid` workgroups (<= its tile count) loop over tiles
// b, b + grid, ...
hipError_t launch_fused_a(const FusedAArgs& a, hipStream_t s);
hipError_t launch_fused_b(const FusedBArgs& a, int grid, hipStream_t s);

}  // namespace brq
