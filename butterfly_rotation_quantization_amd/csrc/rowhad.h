// Row Hadamard path: right-side Hadamard plans (d = 2^k, 16 <= d <= 4096)
// applied to every d-chunk of every row in one pass, for rotate, for
// rotate + quantize + pack, and for dequantize + unrotate.
//
// A workgroup of 256 threads holds 4096 consecutive chunk elements (4096 / d
// chunks), 16 per thread.  The fast Walsh-Hadamard transform runs in rounds:
// in each round the 16 registers of a thread hold elements whose indices
// differ in four (or, in the last round, fewer) bits not yet transformed, the
// radix-2 stages on those bits are butterflies between registers, and an LDS
// transpose brings the next four bits into the registers.  A last transpose
// restores natural order (thread t holds elements 16 t .. 16 t + 15), which
// makes global loads and stores contiguous and keeps quantizer groups on
// consecutive lanes.
//
// The index arithmetic lives here as __host__ __device__ functions so the
// dry run checks exactly what the GPU executes.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kRhThreads = 256;
constexpr int kRhElems = 16;                     // per thread
constexpr int kRhTile = kRhThreads * kRhElems;   // chunk elements per workgroup
constexpr int kRhLds = kRhTile + kRhTile / 16;   // one LDS buffer (padded)
constexpr int kRhBins = 256;                     // codebook search bins

// RH_REQUANT: dequantize, inverse transform, then quantize again with the
// second quantizer (absmax, bits2, group2) -- PolarQuant's downstream chain.
enum RhMode { RH_ROTATE = 0, RH_QUANT = 1, RH_DEQUANT = 2, RH_REQUANT = 3 };

struct RhArgs {
  int log2d;          // chunk length d = 2^log2d
  int mode;           // RhMode
  int64_t rows, n;    // matrix shape, n % d == 0
  int64_t nchunks;    // rows * cpr
  int64_t cpr;        // chunks per row, n / d
  const void* x;      // input [rows][ldx] of type xt (rotate, quantize)
  int xt;
  int64_t ldx;
  void* y;            // output [rows][ldy] of type yt (rotate, dequantize)
  int yt;
  int64_t ldy;
  const float* signs; // d signs (+-1) of the plan, or null
  const float* signs_s;  // the same times scale (with signs)
  int inverse;        // apply M^T: signs after the transform instead of before
  int identity;       // no transform (quantize only): d = 16, no signs, scale 1
  float scale;        // 1 / sqrt(d)
  // quantizer (quantize epilogue, dequantize prologue)
  int qkind, bits, group, nlev;
  float h, sqrt_g;
  float tau[kMaxLevels];   // decision thresholds (codebook)
  float cent[kMaxLevels];  // centroids (codebook dequantize)
  // Codebook search by bins: u = fma(z, bin_s, bin_off) falls in bin
  // floor(u) (clamped to [0, kRhBins)); every threshold's u lies at least
  // 1/64 from an integer and no bin holds two, so the code is the number of
  // thresholds of the bins below plus (z > the bin's own threshold).  The host
  // checks this, records each threshold's bin in tbin, and sets bin_s = 0
  // when no such scaling exists.
  float bin_s, bin_off;
  int tbin[kMaxLevels];
  // The bin table itself, built on the host: bin b holds {its threshold's u
  // (fma(tau, bin_s, bin_off)) or +inf, the number of thresholds in lower
  // bins as the bits of a 32-bit integer}; the kernel compares
  // u = fma(v, k bin_s, bin_off) against it.
  float2 bintab[kRhBins];
  uint8_t* codes;
  const uint8_t* in_codes;
  void* scales;
  const void* in_scales;
  int64_t codes_ld, scales_ld;
  // second quantizer (RH_REQUANT): absmax, output codes and float32 scales
  int bits2, group2;
  float h2;
  int64_t codes_ld2, scales_ld2;
};

static_assert(sizeof(RhArgs) <= 4096, "kernel arguments are limited to 4 KB");

__host__ __device__ constexpr int rh_rounds(int l2d) { return (l2d + 3) / 4; }
// Bits of the element index transformed in round r: [4r, 4r + rh_nnew).
__host__ __device__ constexpr int rh_nnew(int l2d, int r) {
  return (4 * r + 4 < l2d ? 4 * r + 4 : l2d) - 4 * r;
}
// Element-index bit held by register bit q in round r: the top rh_nnew bits of
// the register index are the round's new bits, the others the lowest bits.
__host__ __device__ constexpr int rh_regbit(int l2d, int r, int q) {
  return q < 4 - rh_nnew(l2d, r) ? q : 4 * r + (q - (4 - rh_nnew(l2d, r)));
}
// Index within its chunk of the element that thread cu of the chunk holds in
// register j during round r; the thread index fills the remaining bits in
// increasing order.  Round 0 is natural order: 16 cu + j.
__host__ __device__ inline int rh_elem(int l2d, int r, int cu, int j) {
  int i = 0;
  unsigned used = 0;
  for (int q = 0; q < 4; ++q) {
    const int p = rh_regbit(l2d, r, q);
    i |= ((j >> q) & 1) << p;
    used |= 1u << p;
  }
  int t = cu;
  for (int p = 0; p < l2d; ++p)
    if (!((used >> p) & 1)) {
      i |= (t & 1) << p;
      t >>= 1;
    }
  return i;
}
// Padded LDS slot of element i of chunk cw: one float of padding per 16 spreads
// the strided accesses of the later rounds over the banks.
__host__ __device__ inline int rh_lds(int l2d, int cw, int i) {
  const int x = (cw << l2d) + i;
  return x + (x >> 4);
}

// The same slot split into a per-thread base and a per-register constant.
// The element index of register j in round r is the OR of register j's bits
// (at positions rh_regbit) and the thread's bits (cu at the positions the
// round leaves free, in increasing order: first [4 - nnew, 4r), then
// [4r + nnew, l2d); the chunk cw above l2d).  The two sets of positions are
// disjoint, so x + (x >> 4) of their OR is the sum of the same expression
// for each part; the kernels then address LDS with immediate offsets.
__host__ __device__ constexpr int rh_jbits(int l2d, int r, int j) {
  int i = 0;
  for (int q = 0; q < 4; ++q) i |= ((j >> q) & 1) << rh_regbit(l2d, r, q);
  return i;
}
__host__ __device__ constexpr int rh_lds_off(int l2d, int r, int j) {
  return rh_jbits(l2d, r, j) + (rh_jbits(l2d, r, j) >> 4);
}
__host__ __device__ inline int rh_lds_base(int l2d, int r, int cw, int cu) {
  const int nn = rh_nnew(l2d, r);
  const int A = 4 * r - 4 + nn;  // length of the first free segment
  const int b = (cw << l2d) | ((cu & ((1 << A) - 1)) << (4 - nn)) | ((cu >> A) << (4 * r + nn));
  return b + (b >> 4);
}

// Bin of a scaled value (the kernel's arithmetic, shared with the host check):
// u clamped to [0, kRhBins - 1], then truncated.  The GPU clamps with one
// median-of-three.
__host__ __device__ inline int rh_bin(float u) {
#if defined(__HIP_DEVICE_COMPILE__)
  return (int)__builtin_amdgcn_fmed3f(u, 0.f, (float)(kRhBins - 1));
#else
  const float c = u < 0.f ? 0.f : (u > (float)(kRhBins - 1) ? (float)(kRhBins - 1) : u);
  return (int)c;
#endif
}

__host__ __device__ inline int64_t rh_nwg(const RhArgs& a) {
  const int64_t cpw = kRhTile >> a.log2d;
  return (a.nchunks + cpw - 1) / cpw;
}

// Thread u of workgroup b: chunk cw of the workgroup, thread cu of the chunk,
// global chunk c (live when c < nchunks), its row and the row column of the
// thread's first element in natural order.
struct RhPos {
  int cw, cu;
  int64_t c, row, col0;
  bool live;
};
// Chunk indices fit 31 bits (the host checks nchunks), so the row split is a
// 32-bit division.
__host__ __device__ inline RhPos rh_pos(const RhArgs& a, int64_t b, int u) {
  RhPos p;
  const int tpc = 1 << (a.log2d - 4);
  p.cw = u >> (a.log2d - 4);
  p.cu = u - p.cw * tpc;
  p.c = b * (kRhTile >> a.log2d) + p.cw;
  p.live = p.c < a.nchunks;  // a dead thread reads row 0, columns 0..15 and stores nothing
  const uint32_t c32 = p.live ? (uint32_t)p.c : 0u, cpr = (uint32_t)a.cpr;
  const uint32_t row = c32 / cpr;
  p.row = row;
  p.col0 = p.live ? (int64_t)(c32 - row * cpr) * ((int64_t)1 << a.log2d) + 16 * p.cu : 0;
  return p;
}

// Largest chunk count of one call (chunk indices stay 31-bit).
constexpr int64_t kRhMaxChunks = ((int64_t)1 << 31) - kRhTile;

// Whether the row Hadamard path takes this plan.
inline bool rh_plan_ok(const Plan* p) {
  return p && p->mode == BRQ_HADAMARD && p->d >= 16 && p->d <= 4096 && (p->d & (p->d - 1)) == 0;
}

hipError_t launch_rowhad(const RhArgs& a, hipStream_t s);

bool rh_rotate_supported(const Plan* p, int side, int xt, int yt, int64_t rows, int64_t cols,
                         int64_t ldx, int64_t ldy, const void* x, const void* y);
brq_status rh_rotate(const Plan* p, int inverse, const void* x, int xt, int64_t ldx, void* y,
                     int yt, int64_t ldy, int64_t rows, int64_t cols, hipStream_t s);
bool rh_quant_supported(const Plan* U, const Plan* V, int wt, int64_t m, int64_t n, int64_t ldw,
                        const void* w, const brq_quant* q);
brq_status rh_rqp(const Plan* V, const void* w, int wt, int64_t m, int64_t n, int64_t ldw,
                  const brq_quant* q, uint8_t* codes, void* scales, hipStream_t s);
brq_status rh_dequant(const Plan* V, const uint8_t* codes, const void* scales, const brq_quant* q,
                      int64_t m, int64_t n, void* out, int ot, int64_t ldo, hipStream_t s);
// Dequantize with q_in, inverse transform, quantize + pack with q_out (absmax)
// in one pass; BRQ_ERR_UNSUPPORTED when the plan, shape or alignment does not
// fit the kernel.
brq_status rh_requant(const Plan* V, const uint8_t* codes, const void* scales, const brq_quant* q_in,
                      int64_t m, int64_t n, const brq_quant* q_out, uint8_t* codes_out,
                      void* scales_out, hipStream_t s);
// Quantize + pack with no transform (the quantizer pass after other kernels
// have rotated into a float32 buffer); BRQ_ERR_UNSUPPORTED when the shape or
// alignment does not fit the kernel.
brq_status rh_quant_only(const void* w, int wt, int64_t m, int64_t n, int64_t ldw,
                         const brq_quant* q, uint8_t* codes, void* scales, hipStream_t s);

}  // namespace brq
