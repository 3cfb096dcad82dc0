// Fast path for two-sided plans of the shape U = (bU, 16, 16), V = (bV, 16, 16)
// (bU = 16, bV <= 64): two kernels on MFMA 16x16x4 float32 tiles.  Pass B also
// serves as the tail of longer dense schedules ending in (16, 16) on both
// sides, after stage passes have applied the earlier stages.
//
//  pass A: the first stages U_0 and V_0.  Rows r0*S_U + q (r0 < bU, S_U =
//          256) and columns c0*S_V + p (c0 < bV, S_V the stride of V_0) of
//          one (q, p) pair form a bU x bV matrix X_qp; the pass computes
//          B^U0_q X_qp (B^V0_p)^T for every (q, p) and writes the float32
//          intermediate.  bU is 16 or 32; V may have stages between V_0 and
//          its last two (stage passes apply them in between).  Its products run on
//          f16 MFMA too: the slab of a q is scaled by a power of two that
//          puts its largest magnitude in [2^11, 2^12); 16-bit inputs are then
//          f16 values (hi) and float32 inputs split into hi and lo; V_0's
//          blocks split into (bh, bl); U_0 splits its float32 input like a
//          pass B stage; the output is scaled back.
//  pass B: the remaining radix-16 stages U_1, U_2, V_1, V_2 on a 256 x 256
//          block (rows r0*256 + [0,256), columns c0*256 + [0,256)) held in
//          registers, with one LDS exchange, then the group quantizer and
//          LSB-first packing.  Its products run on f16 MFMA with split
//          operands: the tile is scaled by a power of two so that its
//          largest magnitude lies in [64, 128); every stage splits its
//          float32 data x into hi = f16(x) and lo = f16(x - hi) and uses the
//          blocks split the same way (bh, bl, prepared with the plan), and
//          sums (hi + lo)*bh + (hi + lo)*bl in float32.  Blocks whose
//          entries are all exact in f16 (Hadamard) need (hi + lo)*bh only.
//
// The index arithmetic both kernels use lives here as __host__ __device__
// functions so the host dry run checks exactly what the GPU executes.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kFaWaves = 8;            // pass A: waves per workgroup
constexpr int kFaQC = 8;               // pass A: fewest q values per workgroup (looped; fa_qc)
constexpr int kFbWaves = 16;           // pass B: waves per workgroup
// pass B LDS: the exchange buffer [r1 16][c1h 8][r2 16][c2 16] (swizzled),
// whose first 32 KB hold the tile's 16 V_1 blocks during phase 1, then the
// tile's 16 V_2 blocks.  A staged block is 64 entries of (bh, bh) and, for
// blocks that are not exact in f16, 64 entries of (bl, bl), 16 bytes each at
// fb_vslot.  The 16 waves' tile maxima pass through the exchange buffer
// after the V_1 blocks (free until phase 2).  160 KB in all.
constexpr int kFbXchFloats = 16 * 8 * 16 * 16;
constexpr int kFbV1Off = 0;
constexpr int kFbV1LOff = kFbV1Off + 16 * 256;
constexpr int kFbMaxOff = kFbV1LOff + 16 * 256;
constexpr int kFbV2Off = kFbXchFloats;
constexpr int kFbV2LOff = kFbV2Off + 16 * 256;
constexpr int kFbLdsFloats = kFbV2LOff + 16 * 256;

// Split-f16 blocks of pass B's four stages: block c of a stage is 16 rows x
// 4 quads of 8 halves, entry (j, q) = (bh[j][4q .. 4q+3], bl[j][4q .. 4q+3])
// at halves offset c * kFbBlockHalves + fb_hentry(j, q).
constexpr int kFbBlockHalves = 512;
__host__ __device__ constexpr int fb_hentry(int j, int q) { return (j * 4 + q) * 8; }

struct FusedAArgs {
  const void* w;      // input [m][n], type wt, leading dimension ldw
  int wt;
  int64_t ldw;
  float* ws;          // float32 intermediate [m][n], leading dimension n
  int64_t m, n;
  int bv;             // radix of V_0 (columns)
  int nb;             // 16-blocks spanned by bv
  int ru;             // radix of U_0 (rows): 16 or 32
  int su, sv;         // strides of U_0 (256) and V_0 (d_V / bv)
  int nchunk;         // n / d_V (block-diagonal right side)
  int dv;             // d_V = bv * sv
  // U_0 blocks split into f16 (bh, bl) entries (fa_uhentry), signs folded
  // in; halves between groups (0 = one shared block)
  const uint16_t* u0;
  int64_t u0_gs;
  int u0_exact;       // every U_0 entry exact in f16
  // V_0 blocks split into (bh, bl) entries in fragment order (fa_vhentry),
  // zero-padded to 16 nb, signs folded in
  const uint16_t* v0;
  int64_t v0_gs;
  int64_t u0_n, v0_n; // extents of the block arrays in halves (host checks)
  int qc;             // q values per workgroup (fa_qc)
  int pt;             // p tiles per block of the workgroup order (fa_pt)
};

struct FusedBArgs {
  const float* ws;    // float32 intermediate from pass A (or from stage passes)
  int64_t m, n;
  int nrb;            // 256-row blocks r0: m / 256
  int bv;             // 256-column blocks c0 per d_V (the radix of V_0 after pass A)
  int nchunk, dv;
  // split-f16 blocks (entries as above); strides between groups in halves
  // (0 = one block shared by all groups)
  const uint16_t* u1; int64_t u1_gs;  // U_1, group r0*16 + r2
  const uint16_t* u2; int64_t u2_gs;  // U_2, group r0*16 + r1
  const uint16_t* v1; int64_t v1_gs;  // V_1, group c0*16 + c2
  const uint16_t* v2; int64_t v2_gs;  // V_2, group c0*16 + c1
  int exact;          // every block entry is exact in f16 (bl = 0)
  // quantizer
  int qkind, bits, group, nlev;
  float h, sqrt_g;
  float tau[kMaxLevels];
  uint8_t* codes;
  void* scales;
  int64_t codes_ld, scales_ld;
  int64_t u1_n, u2_n, v1_n, v2_n;  // extents of the block arrays in halves (host checks)
};

// ---- pass A geometry --------------------------------------------------------
//
// A workgroup owns P = 8 * ppw consecutive p (ppw per wave) of one column
// chunk and qc consecutive q (fa_qc).  For each q it stages the input slab
// X[r0 < ru][c0 < bv][P] through LDS (runs of P input elements, at least 64
// bytes), each wave contracts c0 with the V_0 blocks of its own ppw p held in
// registers (ru / 16 row tiles), then r0 with the U_0 block of q, and the
// results leave through a second LDS area as runs of P floats.
//
// V_0 as MFMA steps: chunk ch of 16 columns c0 is one K = 32 product, lane
// (lr, lg) holding x[r0 = lr][c0 = 16 ch + 4 lg + i] (i < 4) as (hi, hi) and
// the block entry (bh, bl) of V[16 nt + lr][16 ch + 4 lg + i] for output tile
// nt; nb = ceil(bv / 16) chunks cover the radix.  (The kernels are
// instantiated per st = ceil(bv / 4), the f32 layout's step count.)

__host__ __device__ constexpr int fa_esz(int wt) { return wt == BRQ_F32 ? 4 : 2; }
// p per wave, as many as the V_0 entries (nb^2 16-byte entries per p and
// lane) leave registers for: 4 for 16-bit input up to nb = 3, else 2;
// float32 input 2, or 1 at nb = 4.
__host__ __device__ constexpr int fa_ppw(int wt, int nb) {
  return wt == BRQ_F32 ? (nb >= 4 ? 1 : 2) : (nb >= 4 ? 2 : 4);
}
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
// row (j % ru), column block cb = j / ru.  Columns past the radix repeat the
// last one, so every wave issues the same fixed number of instructions.
__host__ __device__ constexpr int fa_ncb(int runs_per_inst, int st) {
  return (4 * st + runs_per_inst - 1) / runs_per_inst;
}
__host__ __device__ constexpr int fa_ki(int wt, int st, int ru) {
  return ru / 8 * fa_ncb(64 / fa_ipr(wt, fa_nb_of_steps(st)), st);
}
// Output stores of one 16-column tile nt: ru rows x 16 columns of P / 4
// float4s, lpr = P / 4 lanes per run, as kq_nt instructions per wave.
__host__ __device__ constexpr int fa_kq_nt(int wt, int st, int ru) {
  return ru * fa_p(wt, fa_nb_of_steps(st)) / 128;
}
struct FaSlot {
  int r0, c0;
};
// c_first: first column of the range (0 for slab loads, 16 nt for the
// stores of output tile nt).
__host__ __device__ inline FaSlot fa_slot(int lpr, int w, int k, int lane, int bv, int c_first, int ru) {
  const int j = w + 8 * k;
  FaSlot x;
  x.r0 = j % ru;
  const int c0 = c_first + (j / ru) * (64 / lpr) + lane / lpr;
  x.c0 = c0 < bv ? c0 : bv - 1;
  return x;
}

struct FaGeom {
  int P, ppw, esz, ipr;
  int max_off;     // byte offset of the 8 waves' slab maxima (after the output area)
  int rsb;         // slab: bytes between runs (c0), P*esz + 8
  int rowb;        // slab: bytes between r0 rows; rowb / 8 odd
  int rowo;        // output area: floats between r0 rows; rowo / 4 odd
  int slab_bytes;  // ru * rowb, rounded up to 16
  int out_floats;  // ru * rowo
  int items;       // 16-byte input items per q: ru * bv * ipr
  int quads;       // float4 outputs per q: ru * bv * P / 4
};

// The pads make the 16 lanes of a row group (16 different r0, same c0) hit
// distinct LDS banks on the 8-byte slab reads and the 16-byte output writes.
__host__ __device__ inline FaGeom fa_geom(int wt, int nb, int bv, int ru) {
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
  g.slab_bytes = (ru * g.rowb + 15) / 16 * 16;
  g.out_floats = ru * g.rowo;
  g.items = ru * bv * g.ipr;
  g.quads = ru * bv * g.P / 4;
  g.max_off = g.slab_bytes + g.out_floats * (int)sizeof(float);
  return g;
}

__host__ __device__ inline int fa_lds_bytes(const FaGeom& g) { return g.max_off + kFaWaves * 4; }

// Slab scale of pass A: 2^k with k = fa_scale_shift(M) puts the largest
// magnitude M of the slab in [2^11, 2^12) (M below 2^-126 or zero: k = 138,
// which keeps every value below 2^12).  A V_0 block row has norm at most
// 1 + 1e-3 (the host checks), so V_0's outputs, which U_0 splits into f16,
// stay below 8 * 1.001 * 2^12 < 65504 for radices up to 64.
__host__ __device__ inline int fa_scale_shift(uint32_t mbits) { return 138 - (int)((mbits >> 23) & 0xff); }

// q values per workgroup: 32 or 16 when su allows it and the grid still
// gives each of the cus CUs a workgroup and splits into 8 equal XCD shares,
// else kFaQC.  A workgroup loads its V_0 entries and pays its start-up
// latency once for all its q, and with fewer q groups each XCD reads the V_0
// entries of fewer of them.
inline int fa_qc(int64_t nwg8, int su, int cus) {
  for (int qc = 32; qc > kFaQC; qc /= 2) {
    const int64_t n = nwg8 * kFaQC / qc;
    if (su % qc == 0 && n >= cus && n % 8 == 0) return qc;
  }
  return kFaQC;
}

struct FaTile {
  int p0, q0, chunk;
};

__host__ __device__ inline int64_t fa_nwg(const FusedAArgs& a) {
  return (int64_t)(a.sv / fa_p(a.wt, a.nb)) * (a.su / a.qc) * a.nchunk;
}

// Workgroup b -> (p range, q range, column chunk).  Workgroup b goes to XCD
// b mod 8 and takes position lin of that XCD's share (the grid is a multiple
// of 8).  In lin order the p tiles run in blocks of a.pt (fa_pt), then the q
// groups, then the blocks, then the chunks: an XCD's workgroups share every
// input line they touch in its L2, and each XCD reads the V_0 entries of
// only its own p tiles.
//
// p tiles per block: grids of at least four workgroups per CU take the
// tiles that share 128-byte input lines (two 64-byte runs), so an XCD holds
// few p tiles' V_0 entries at a time; smaller grids take 512 contiguous
// bytes of a row per q.  Measured on the 16-bit weights: the 8192-row weight
// with radix 7 (1024 workgroups) ran pass A in 487 us with pairs against 499
// with 512-byte blocks; the 256-workgroup grids (4096 and 11008 columns)
// were 4% slower with pairs.
inline int fa_pt(const FusedAArgs& a, int64_t nwg, int cus) {
  const int P = fa_p(a.wt, a.nb), run = P * fa_esz(a.wt), npt = a.sv / P;
  const int bytes = nwg >= 4 * (int64_t)cus ? 128 : 512;
  const int pt = run >= bytes ? 1 : bytes / run;
  return pt < npt ? pt : npt;
}
__host__ __device__ inline FaTile fa_tile(const FusedAArgs& a, int64_t b, int64_t nwg) {
  const int P = fa_p(a.wt, a.nb), pt = a.pt, nqg = a.su / a.qc;
  const int64_t per_xcd = nwg / 8;
  const int64_t lin = (b % 8) * per_xcd + b / 8;
  const int64_t per_block = (int64_t)pt * nqg, per_chunk = (int64_t)(a.sv / P) * nqg;
  const int64_t in_chunk = lin % per_chunk;
  const int64_t blk = in_chunk / per_block, r = in_chunk % per_block;
  FaTile t;
  t.p0 = (int)(blk * pt + r % pt) * P;
  t.q0 = (int)(r / pt) * a.qc;
  t.chunk = (int)(lin / per_chunk);
  return t;
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
__host__ __device__ inline int64_t fa_row(const FusedAArgs& a, int r0, int q) { return (int64_t)r0 * a.su + q; }
__host__ __device__ inline int64_t fa_col(const FusedAArgs& a, int chunk, int c0, int p) {
  return (int64_t)chunk * a.dv + (int64_t)c0 * a.sv + p;
}
// Halves offset of the U_0 entry (row j, quad q) within a ru x ru block
// (2 ru^2 halves): (bh, bl) of U[j][4 q .. 4 q + 3].
__host__ __device__ constexpr int fa_uhentry(int ru, int j, int q) { return (j * (ru / 4) + q) * 8; }
// Halves offset of the fragment-order V_0 entry (nt, lr, lg, ch) within a
// group (512 nb^2 halves): the nb chunks of one (nt, lane) are contiguous.
__host__ __device__ inline int64_t fa_vhentry(int nb, int nt, int lr, int lg, int ch) {
  return ((((int64_t)nt * 16 + lr) * 4 + lg) * nb + ch) * 8;
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
// fixed) the quad index takes r2 % 4 XOR r1 % 4 in its low two bits and
// c2 / 4 XOR r2 / 4 XOR r1 / 4 in its high two.  Every 8 and every 16
// consecutive lanes then hit distinct bank groups both on the phase-1
// writes (lanes over r1 at fixed c1h, r2, c2 / 4) and on the phase-2 reads
// and write-backs (lanes over r2 at fixed r1, c1h, c2 / 4).
__host__ __device__ inline int fb_xch(int r1, int c1h, int r2, int c2) {
  const int hi = (r1 * 8 + c1h) * 4 + (r2 >> 2);
  const int lo = ((r2 & 3) ^ (r1 & 3)) | ((((c2 >> 2) ^ (r2 >> 2) ^ (r1 >> 2)) & 3) << 2);
  return (hi * 16 + lo) * 4 + (c2 & 3);
}

// Float offset of quad q (columns 4q .. 4q + 3) of row j of a 16 x 16 V block
// staged in LDS.  The quad index is XORed with ((j >> 1) & 3) ^ ((j >> 3) & 1),
// so that the 16-byte reads of V_1 (lanes lr over rows fb_sigma(lr)) and of
// V_2 (lanes over rows lr), at a fixed quad, fall on distinct bank groups
// for every 8 and every 16 consecutive lanes; unswizzled, the 64-byte row
// stride put the lanes of a read on two bank groups.
__host__ __device__ inline int fb_vslot(int j, int q) {
  return (j * 4 + (q ^ (((j >> 1) & 3) ^ ((j >> 3) & 1)))) * 4;
}

// Pass B's quantizer: lane (lr, lg) codes 32 consecutive columns of one row,
// so a group of g columns spans g / 32 lanes of consecutive lg; the first of
// them stores the group's statistic.
__host__ __device__ constexpr bool fb_scale_lane(int lg, int g) { return (lg & (g / 32 - 1)) == 0; }

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

// Tile scale of pass B: 2^k with k = fb_scale_shift(M) puts the largest
// magnitude M of a tile in [64, 128) (k = 127 for M below 2^-121 or zero).
// The blocks' rows have norm at most 1 + 1e-3 (the host checks), so no value
// of the four stages exceeds 4^4 * 1.004 * 128 < 65504.
__host__ __device__ inline int fb_scale_shift(uint32_t mbits) {
  const int e = (int)((mbits >> 23) & 0xff);
  const int s = 260 - e;
  return (s > 254 ? 254 : s) - 127;
}
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
