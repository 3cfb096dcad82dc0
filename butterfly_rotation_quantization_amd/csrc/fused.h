// Fast path for two-sided plans of the shape U = (bU, 16, 16), V = (bV, 16, 16)
// (bU = 16, bV <= 64): two kernels on MFMA 16x16x4 float32 tiles.  Pass B also
// serves as the tail of longer dense schedules ending in (16, 16) on both
// sides, after stage passes have applied the earlier stages.
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

constexpr int kFaWaves = 8;            // pass A: waves per workgroup
constexpr int kFaQC = 8;               // pass A: q values per workgroup (looped)
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
  int nb;             // 16-blocks spanned by bv
  int nchunk;         // n / d_V (block-diagonal right side)
  int dv;             // d_V = bv * 256
  const float* u0;    // U_0 blocks [256][16][16] (or one shared block), signs folded in
  int64_t u0_gs;      // float stride between groups (0 = shared)
  const float* v0f;   // V_0 blocks in fragment order [256][nb][16][4][4nb] (or one), signs folded in
  int64_t v0_gs;
  uint32_t bv_magic;  // floor(2^32 / bv) + 1: i / bv = (i * bv_magic) >> 32 for the i used
  int64_t u0_n, v0_n; // float extents of the block arrays (host checks)
};

struct FusedBArgs {
  const float* ws;    // float32 intermediate from pass A (or from stage passes)
  int64_t m, n;
  int nrb;            // 256-row blocks r0: m / 256
  int bv;             // 256-column blocks c0 per d_V (the radix of V_0 after pass A)
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
//
// A workgroup owns P = 8 * ppw consecutive p (ppw per wave) of one column
// chunk and kFaQC consecutive q.  For each q it stages the input slab
// X[r0 < 16][c0 < bv][P] through LDS (runs of P input elements, at least 64
// bytes), each wave contracts c0 with the V_0 blocks of its own ppw p held in
// registers, then r0 with the U_0 block of q, and the results leave through a
// second LDS area as runs of P floats.
//
// V_0 as MFMA steps: step s contracts c0 = 4s + lg (lane group lg), so
// ceil(bv / 4) steps cover the radix and the block fragment of step s and
// output tile nt is V[16 nt + lr][4 s + lg].

__host__ __device__ constexpr int fa_esz(int wt) { return wt == BRQ_F32 ? 4 : 2; }
// p per wave: 4, or 2 where the blocks (nb = 4) or the float32 slab would not fit.
__host__ __device__ constexpr int fa_ppw(int wt, int nb) { return (wt == BRQ_F32 || nb == 4) ? 2 : 4; }
__host__ __device__ constexpr int fa_p(int wt, int nb) { return 8 * fa_ppw(wt, nb); }
// 16-byte input items per run of P elements
__host__ __device__ constexpr int fa_ipr(int wt, int nb) { return fa_p(wt, nb) * fa_esz(wt) / 16; }

// MFMA steps of V_0 (4 columns c0 each) and 16-blocks spanned by the radix.
__host__ __device__ constexpr int fa_steps(int bv) { return (bv + 3) / 4; }
__host__ __device__ constexpr int fa_nb_of_steps(int st) { return (st + 3) / 4; }
// Slab loads and output stores take one row r0 and 64 / lpr consecutive
// columns c0 per wave instruction (lpr lanes per run of P elements: ipr for
// loads, P / 4 for stores): lane l holds part l % lpr of column
// cb * (64 / lpr) + l / lpr.  Instruction k of wave w is slot j = w + 8 k:
// row (j % 16), column block cb = j / 16.  Columns past the radix repeat the
// last one, so every wave issues the same fixed number of instructions.
__host__ __device__ constexpr int fa_ncb(int runs_per_inst, int st) {
  return (4 * st + runs_per_inst - 1) / runs_per_inst;
}
__host__ __device__ constexpr int fa_ki(int wt, int st) {
  return 2 * fa_ncb(64 / fa_ipr(wt, fa_nb_of_steps(st)), st);
}
// Output stores of one 16-column tile nt: 16 rows x 16 columns of P / 4
// float4s, lpr = P / 4 lanes per run, as kq_nt instructions per wave.
__host__ __device__ constexpr int fa_kq_nt(int wt, int st) { return fa_p(wt, fa_nb_of_steps(st)) / 8; }
struct FaSlot {
  int r0, c0;
};
// c_first: first column of the range (0 for slab loads, 16 nt for the
// stores of output tile nt).
__host__ __device__ inline FaSlot fa_slot(int lpr, int w, int k, int lane, int bv, int c_first) {
  const int j = w + 8 * k;
  FaSlot x;
  x.r0 = j % 16;
  const int c0 = c_first + (j / 16) * (64 / lpr) + lane / lpr;
  x.c0 = c0 < bv ? c0 : bv - 1;
  return x;
}

struct FaGeom {
  int P, ppw, esz, ipr;
  int rsb;         // slab: bytes between runs (c0), P*esz + 8
  int rowb;        // slab: bytes between r0 rows; rowb / 8 odd
  int rowo;        // output area: floats between r0 rows; rowo / 4 odd
  int slab_bytes;  // 16 * rowb, rounded up to 16
  int out_floats;  // 16 * rowo
  int items;       // 16-byte input items per q: 16 * bv * ipr
  int quads;       // float4 outputs per q: 16 * bv * P / 4
};

// The pads make the 16 lanes of a row group (16 different r0, same c0) hit
// distinct LDS banks on the 8-byte slab reads and the 16-byte output writes.
__host__ __device__ inline FaGeom fa_geom(int wt, int nb, int bv) {
  FaGeom g;
  g.ppw = fa_ppw(wt, nb);
  g.esz = fa_esz(wt);
  g.P = 8 * g.ppw;
  g.ipr = g.P * g.esz / 16;
  g.rsb = g.P * g.esz + 8;
  g.rowb = bv * g.rsb;
  if (((g.rowb / 8) & 1) == 0) g.rowb += 8;
  g.rowo = bv * g.P;
  if (((g.rowo / 4) & 1) == 0) g.rowo += 4;
  g.slab_bytes = (16 * g.rowb + 15) / 16 * 16;
  g.out_floats = 16 * g.rowo;
  g.items = 16 * bv * g.ipr;
  g.quads = 16 * bv * g.P / 4;
  return g;
}

__host__ __device__ inline int fa_lds_bytes(const FaGeom& g) {
  return g.slab_bytes + g.out_floats * (int)sizeof(float);
}

// Workgroup b -> (p range, q chunk, column chunk).  Workgroups are dealt to
// the 8 XCDs round robin (b % 8); consecutive slots of one XCD walk the p
// ranges first, so workgroups sharing input rows share that XCD's L2.
struct FaTile {
  int p0, q0, chunk;
};

__host__ __device__ inline int64_t fa_nwg(const FusedAArgs& a) {
  return (int64_t)(256 / fa_p(a.wt, a.nb)) * (256 / kFaQC) * a.nchunk;
}

__host__ __device__ inline FaTile fa_tile(const FusedAArgs& a, int64_t b, int64_t nwg) {
  const int P = fa_p(a.wt, a.nb);
  const int64_t per_xcd = nwg / 8;
  const int64_t lin = (b % 8) * per_xcd + b / 8;
  FaTile t;
  t.p0 = (int)(lin % (256 / P)) * P;
  const int64_t rest = lin / (256 / P);
  t.q0 = (int)(rest % (256 / kFaQC)) * kFaQC;
  t.chunk = (int)(rest / (256 / kFaQC));
  return t;
}

// i / bv without a division instruction (exact for the ranges the host checks).
__host__ __device__ inline int fa_div_bv(const FusedAArgs& a, int i) {
  return (int)(((uint64_t)(uint32_t)i * a.bv_magic) >> 32);
}

// Byte offset of input item (r0, c0, o) in the slab (8-byte aligned).
__host__ __device__ inline int fa_slab_item(const FaGeom& g, int r0, int c0, int o) {
  return r0 * g.rowb + c0 * g.rsb + 16 * o;
}
// Byte offset of the ppw elements (r0, c0, [ppw*w, ppw*w + ppw)) in the slab.
__host__ __device__ inline int fa_slab_read(const FaGeom& g, int r0, int c0, int w) {
  return r0 * g.rowb + c0 * g.rsb + g.ppw * w * g.esz;
}
// Float offset of output (r0', c0', p_local) in the output area.
__host__ __device__ inline int fa_out(const FaGeom& g, int r0, int c0, int pl) {
  return r0 * g.rowo + c0 * g.P + pl;
}
// Global element (row, col) of (r0, q) x (chunk, c0, p).
__host__ __device__ inline int64_t fa_row(int r0, int q) { return (int64_t)r0 * 256 + q; }
__host__ __device__ inline int64_t fa_col(const FusedAArgs& a, int chunk, int c0, int p) {
  return (int64_t)chunk * a.dv + (int64_t)c0 * 256 + p;
}
// Fragment-order V_0 block index of (group, nt, lr, lg, s): the 4 nb steps of
// one (nt, lane) are contiguous.
__host__ __device__ inline int64_t fa_vfrag(int nb, int nt, int lr, int lg, int s) {
  return (((int64_t)nt * 16 + lr) * 4 + lg) * (4 * nb) + s;
}

// ---- pass B geometry --------------------------------------------------------

struct FbTile {
  int r0, c0, chunk;
};

__host__ __device__ inline int64_t fb_nwg(const FusedBArgs& a) {
  return (int64_t)a.nrb * a.bv * a.nchunk;
}

__host__ __device__ inline FbTile fb_tile(const FusedBArgs& a, int64_t b) {
  FbTile t;
  t.r0 = (int)(b % a.nrb);
  const int64_t rest = b / a.nrb;
  t.c0 = (int)(rest % a.bv);
  t.chunk = (int)(rest / a.bv);
  return t;
}

// Exchange slot of element (r1, c1h, r2, c2), c1h = c1 - 8 h.  Each float4
// holds four consecutive c2; within every 16 float4s (r1, c1h and r2 / 4
// fixed) the quad index (r2 % 4, c2 / 4) is XORed with r1 and r2 / 4.  The 16
// lanes of a row group then hit 16 different bank groups both on the phase-1
// writes (lanes over r1 at fixed c1h, r2, c2 / 4) and on the phase-2 reads
// (lanes over r2 at fixed r1, c1h, c2 / 4).
__host__ __device__ inline int fb_xch(int r1, int c1h, int r2, int c2) {
  const int hi = (r1 * 8 + c1h) * 4 + (r2 >> 2);
  const int lo = (((r2 & 3) * 4 + (c2 >> 2)) ^ (r2 >> 2) ^ r1) & 15;
  return (hi * 16 + lo) * 4 + (c2 & 3);
}

// Row order of the V_1 products: output tile row n holds c1' = fb_sigma(n),
// so MFMA result register j of lane group lg holds c1' = lg + 4 j and the
// exchange half h (c1' in [8h, 8h + 8)) is registers 2h and 2h + 1 of every
// lane.
__host__ __device__ inline int fb_sigma(int n) { return (n >> 2) + 4 * (n & 3); }

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

// Pass B alone as the tail of a two-sided transform whose last two stages are
// radix 16 on both sides (dense blocks, m and d_V multiples of 256): the
// caller has applied every earlier stage into the float32 workspace `ws`;
// pass B applies U_{m-2}, U_{m-1}, V_{m-2}, V_{m-1}, quantizes and packs.
bool fused_tail_supported(const Plan* U, const Plan* V, int64_t m, int64_t n, const brq_quant* q);
brq_status fused_tail_rqp(const Plan* U, const Plan* V, const float* ws, int64_t m, int64_t n,
                          const brq_quant* q, uint8_t* codes, void* scales, hipStream_t s);

// Kernel launchers (fused_kernels.hip; the dry-run build walks their indices).
// Pass B is persistent: `grid` workgroups (<= its tile count) loop over tiles
// b, b + grid, ...
hipError_t launch_fused_a(const FusedAArgs& a, hipStream_t s);
hipError_t launch_fused_b(const FusedBArgs& a, int grid, hipStream_t s);

}  // namespace brq
