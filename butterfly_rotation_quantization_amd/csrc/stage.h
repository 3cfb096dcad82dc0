// Stage pass: one stage of one side applied to the whole matrix in one launch.
//
// The multi-stage tile pass fuses several stages per tile, which needs a whole
// group product of a line in one workgroup; with few lines (online activation
// rotation at decode time: 1 to a few hundred rows) that leaves a handful of
// workgroups for the whole GPU.  The stage pass instead splits the groups of
// one stage over the workgroups, so every stage has d / b groups of
// parallelism whatever the row count, and a plan of m stages takes m launches
// (the intermediate stays in a float32 buffer that is updated in place).
//
// Stage arithmetic ([HARP] technical summary 2.1): group c = hi * S + lo of a
// stage with radix b and stride S holds the elements hi * b * S + k * S + lo
// (k < b) of a d-chunk, and y_j = sum_k B_c[j][k] x_k.
//
// A workgroup takes `gw` consecutive groups (global index over all chunks)
// and up to kSpLines lines (rows for the right side, columns for the left).
// Thread (g, j) keeps row j of block B_g in registers and produces output j of
// group g for every line of the tile; the tile goes through LDS on the way in
// and out so global loads and stores are coalesced.
//
// The index arithmetic lives here as __host__ __device__ functions so the dry
// run checks exactly what the GPU executes.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kSpThreads = 256;
constexpr int kSpLines = 32;        // lines per tile
constexpr int kSpLineFloats = 256;  // gw * bs <= 256 floats of a line in LDS

struct SpArgs {
  int side;              // 0: right (lines are rows), 1: left (lines are columns)
  int b;                 // radix of the stage
  int bp;                // threads per group: b rounded up to a power of two
  int bs;                // LDS floats per group: b rounded up to a multiple of 4
  int gw;                // groups per tile (kSpThreads / bp)
  int mode;              // BRQ_HADAMARD, BRQ_SHARED, BRQ_PER_GROUP
  int64_t S;             // stride of the stage along the transformed axis
  int64_t d;             // plan dimension
  int64_t ngc;           // groups per chunk, d / b
  int64_t ngroups;       // groups over all chunks
  int64_t lines;         // rows (right side) or columns (left side)
  const float* blk;      // blocks of the stage ([group][j][k], or one [j][k]); null: Hadamard
  int blk_vec;           // blk 16-byte aligned and b % 4 == 0: block rows load as float4
  float hscale;          // 1 / sqrt(b) for Hadamard blocks
  const float* sign_in;  // signs applied when loading (first forward stage), or null
  const float* sign_out; // signs applied when storing (last inverse stage), or null
  const void* src;
  int src_t;
  int64_t ld_src;
  void* dst;
  int dst_t;
  int64_t ld_dst;
  // Optional second stage in the same tile (right side): the pair (16,
  // S = 16), (16, 1) forward, or (16, 1), (16, S = 16) inverse (inv2), with
  // gw = 16 groups, one block of 256 consecutive positions per line.
  // Forward, the first stage leaves output (g, j) at slot (j, g), i.e. in
  // position order, the second stage's group g2 reads the consecutive slots
  // (g2, k2) and writes output (g2, j2) at slot (j2, g2), the first stage's
  // slot of that position, where the store phase reads it.  Inverse, the
  // first stage's groups are the rows of the 16 x 16 position block, so its
  // output (g, j) stays at slot (g, j) (position order already); the second
  // stage's group g2 is the column g2, members at slots (k2, g2), and it
  // writes output j2 at slot (j2, g2), again that position's slot.
  int b2;             // 16, or 0 for a single stage
  int inv2;           // the pair is the inverse one
  // right side: lines per tile, kSpLines, kSpLinesFew or kSpLinesTiny (more
  // workgroups, each lighter); the left side always takes kSpLines
  int tile_lines;
  const float* blk2;  // its blocks ([group][j][k] over the chunk's d / b2 groups, or one)
  // right side, float32 source: the source is the sum of nparts arrays
  // part_stride elements apart (split partial sums of a product), added part
  // by part into four running sums, part p into sum p mod 4, then (s0 + s1) +
  // (s2 + s3); nparts 0 or 1: one array
  int nparts;
  int64_t part_stride;
};

// Float offset of row j2 of the second stage's block for local group g2 of
// the tile whose first group is gid0: the tile is the 256-position block hi
// of its chunk (16 first-stage groups per tile in both pair orders), and the
// second stage's group is hi * 16 + g2.
__host__ __device__ inline int64_t sp_block_row2(const SpArgs& a, int64_t gid0, int g2, int j2) {
  const int64_t hi = ((uint32_t)gid0 % (uint32_t)a.ngc) / (uint32_t)a.gw;
  const int64_t c2 = a.mode == BRQ_PER_GROUP ? hi * a.b + g2 : 0;
  return (c2 * a.b2 + j2) * a.b2;
}

__host__ __device__ inline int64_t sp_group_tiles(const SpArgs& a) {
  return (a.ngroups + a.gw - 1) / a.gw;
}
constexpr int kSpLinesFew = 8;
constexpr int kSpLinesTiny = 4;       // right side, up to kSpTinyRows rows
constexpr int kSpTinyRows = 16;
__host__ __device__ inline int sp_tl(const SpArgs& a) {
  if (a.side != 0) return kSpLines;
  return a.tile_lines == kSpLinesTiny ? kSpLinesTiny : (a.tile_lines == kSpLinesFew ? kSpLinesFew : kSpLines);
}
__host__ __device__ inline int64_t sp_line_tiles(const SpArgs& a) {
  return (a.lines + sp_tl(a) - 1) / sp_tl(a);
}
// The GPU hands workgroup i to XCD i % kXcds, and each XCD has its own L2.
// Workgroup bid takes logical tile xcd_order(bid, n), which numbers the
// tiles XCD by XCD, so consecutive logical tiles run on one XCD at about the
// same time and share its L2 lines (tiles of 64-byte runs split 128-byte lines
// with their neighbours).  A bijection of [0, n) for any n.
constexpr uint32_t kXcds = 8;
__host__ __device__ inline uint32_t xcd_order(uint32_t bid, uint32_t n) {
  const uint32_t q = n / kXcds, r = n % kXcds, x = bid % kXcds, s = bid / kXcds;
  return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}
__host__ __device__ inline int64_t sp_blocks(const SpArgs& a) {
  return sp_group_tiles(a) * sp_line_tiles(a);
}
// Tile of workgroup bid (a one-dimensional grid of sp_blocks workgroups).
// Logical tiles run along the groups on the right side (the next groups of
// the same rows) and along the lines on the left side (the next columns of
// the same rows): consecutive addresses either way.
__host__ __device__ inline void sp_tile_of_block(const SpArgs& a, uint32_t bid, int64_t& gt,
                                                 int64_t& lt) {
  const uint32_t t = xcd_order(bid, (uint32_t)sp_blocks(a));
  const uint32_t nf = (uint32_t)(a.side ? sp_line_tiles(a) : sp_group_tiles(a));
  const uint32_t slow = t / nf, fast = t - slow * nf;
  gt = a.side ? slow : fast;
  lt = a.side ? fast : slow;
}

// Position along the transformed axis of member k of group gid (global over
// chunks), in 32-bit arithmetic: the host keeps every position below 2^31.
__host__ __device__ inline int64_t sp_pos(const SpArgs& a, int64_t gid, int k) {
  const uint32_t gi = (uint32_t)gid, ngc = (uint32_t)a.ngc, S = (uint32_t)a.S;
  const uint32_t chunk = gi / ngc;
  const uint32_t c = gi - chunk * ngc;
  const uint32_t hi = c / S;
  const uint32_t lo = c - hi * S;
  return (int64_t)(chunk * (uint32_t)a.d + (hi * (uint32_t)a.b + (uint32_t)k) * S + lo);
}

// Float offset of row j of the block of group gid in the stage's block array
// (per-group blocks are indexed by the group within its chunk).
__host__ __device__ inline int64_t sp_block_row(const SpArgs& a, int64_t gid, int j) {
  const int64_t c = a.mode == BRQ_PER_GROUP ? (int64_t)((uint32_t)gid % (uint32_t)a.ngc) : 0;
  return (c * a.b + j) * a.b;
}

// Element offset of (line, position) in a matrix with leading dimension ld.
__host__ __device__ inline int64_t sp_off(const SpArgs& a, int64_t line, int64_t pos, int64_t ld) {
  return a.side == 0 ? line * ld + pos : pos * ld + line;
}

// Member (g, k) of a tile's inner index q (0 <= q < gw * b; larger q give
// members the callers skip).  The right side's
// load and store loops give thread q one member and walk the lines, so
// consecutive q must be consecutive positions: k fastest when S = 1 (group
// hi holds positions hi * b + k), group fastest otherwise (consecutive lo).
// The left side's loops walk q with the lines fastest across threads, and any
// order does.
__host__ __device__ inline void sp_member(const SpArgs& a, int q, int& g, int& k) {
  const bool kfast = a.side == 1 || a.S == 1;  // selects, not branches: g and k stay in registers
  const int div = kfast ? a.b : a.gw;
  const int hi = q / div, lo = q - hi * div;
  g = kfast ? hi : lo;
  k = kfast ? lo : hi;
}

// LDS slot of (line, group, member) in one tile buffer.  Right side: line
// major, so the lanes of a load or store (one member each) are consecutive
// slots.  Left side: member major with lines fastest (kSpLinePad floats per
// member), because there the lanes of a load or store span the lines; the
// products then read four lines per float4.
constexpr int kSpLinePad = kSpLines + 4;
constexpr int kSpBufFloats = kSpLineFloats * kSpLinePad;  // the larger of the two layouts
__host__ __device__ inline int sp_lds(const SpArgs& a, int l, int g, int k) {
  return a.side == 0 ? l * kSpLineFloats + g * a.bs + k : (g * a.bs + k) * kSpLinePad + l;
}

hipError_t launch_stage(const SpArgs& a, hipStream_t s);

// ---- Left-side stages by whole rows ------------------------------------------
//
// On the left side the members of a group are whole matrix rows: group
// c = hi * S + lo maps rows hi * b * S + k * S + lo (k < b) to the same rows,
// Y[j][:] = sum_k B_c[j][k] X[k][:].  This kernel gives a workgroup one group
// and kSrThreads * vec consecutive columns; thread t owns vec columns and keeps
// its b x vec inputs in registers, so every load and store is a contiguous
// run of a row and no LDS is needed.  All threads of a workgroup share one
// block, whose entries are therefore uniform and come through the scalar
// cache.  Radices 2 .. 64 that are powers of two take it (Hadamard blocks up
// to 16, the canonical radices); the pointers, leading dimensions and column
// count must allow vec-element accesses, and one side must be float32.
constexpr int kSrThreads = 256;
__host__ __device__ constexpr int sr_vec(int b) { return b <= 16 ? 4 : (b >= 64 ? 1 : 64 / b); }
__host__ __device__ inline int64_t sr_col_tiles(const SpArgs& a) {
  const int64_t w = (int64_t)kSrThreads * sr_vec(a.b);
  return (a.lines + w - 1) / w;
}
// Group and column tile of workgroup bid; column tiles run fastest, so
// consecutive workgroups read consecutive runs of the same rows.
__host__ __device__ inline void sr_tile_of_block(uint32_t bid, uint32_t nct, uint32_t& gid,
                                                 uint32_t& ct) {
  gid = bid / nct;
  ct = bid - gid * nct;
}
// First column of thread t in column tile ct.
__host__ __device__ inline int64_t sr_col(uint32_t ct, int t, int vec) {
  return ((int64_t)ct * kSrThreads + t) * vec;
}
bool sr_supported(const SpArgs& a);
hipError_t launch_stage_rows(const SpArgs& a, hipStream_t s);

// ---- Right-side stages of radix <= 8 by groups in lanes ------------------------
//
// With b <= 8 a whole block (b^2 <= 64 floats) fits in registers, so a lane
// can own one group: lane l of a workgroup takes group c = hi * S + lo0 + l
// of one chunk, keeps B_c and its signs in registers, and walks rows.  The
// groups of a workgroup are 64 consecutive lo, so each member k is a
// 256-byte run of a row (64 consecutive positions) and every load and store
// is coalesced; the four waves take every fourth row of the workgroup's row
// range.  The blocks of the workgroup's 64 groups are contiguous in the
// block array and pass through LDS once.  S must be a multiple of 64, and
// at least 8 rows (below, the tile kernel spreads wider).  Radix 16 takes
// the same path with a quarter of each block per wave (stage_lanes.hip).
constexpr int kSlThreads = 256;
constexpr int kSlLanes = 64;   // groups per workgroup
struct SlGeom {
  int64_t lo_tiles;  // workgroups along the groups: nchunk * (d / (b S)) * S / 64
  int64_t row_tiles; // workgroups along the rows
  int rows_per;      // rows per workgroup (a multiple of 4)
};
__host__ __device__ inline SlGeom sl_geom(const SpArgs& a, int rows_per) {
  SlGeom g;
  g.lo_tiles = a.ngroups / kSlLanes;
  g.rows_per = rows_per;
  g.row_tiles = (a.lines + rows_per - 1) / rows_per;
  return g;
}
// Group (global over chunks) of lane l of lo tile t: the tile's 64 groups are
// consecutive group indices.
__host__ __device__ inline int64_t sl_group(int64_t t, int l) { return t * kSlLanes + l; }
bool sl_supported(const SpArgs& a);
int sl_rows_per(const SpArgs& a);
hipError_t launch_stage_lanes(const SpArgs& a, int rows_per, hipStream_t s);

// Host side (stage_host.cpp).  sp_shape_ok: the stage pass can run the plan
// on this shape; sp_rotate_supported: it is also the faster choice.
bool sp_shape_ok(const Plan* p, int side, int64_t rows, int64_t cols);
bool sp_rotate_supported(const Plan* p, int side, int64_t rows, int64_t cols);
brq_status sp_rotate(const Plan* p, int side, int inverse, const void* x, int xt, int64_t ldx,
                     void* y, int yt, int64_t ldy, int64_t rows, int64_t cols, void* ws,
                     size_t ws_bytes, hipStream_t s, hipError_t* herr);
// ---- Two consecutive right-side stages in one launch, for few rows ----------
//
// Stages (b_o, S_o) and (b_i, S_i) next to each other in a schedule have
// S_o = b_i S_i, so position hi (b_o b_i S_i) + a S_o + b S_i + lo of a chunk
// is element (a, b) of the closed set (hi, lo): the outer stage mixes a for
// each b, the inner one b for each a.  A workgroup takes sets = 256 / (b_o
// b_i) consecutive lo of one hi; thread (set, g, j)
// makes output j of group g of each stage, its block rows loaded up front,
// the set's elements in LDS between the two stages, kP2Lines rows per
// workgroup (more rows: more workgroups).  Forward runs the outer
// stage first, inverse (transposed blocks) the inner one.  Used up to
// kP2MaxLines rows, where the two stages would otherwise be two tile-kernel
// launches.
constexpr int kP2Lines = 4;
constexpr int kP2MaxLines = 32;
struct P2Args {
  int bo, bi;              // radices of the outer and inner stage (bo * bi <= 256, each <= 16)
  int64_t Si;              // inner stride (outer: bo's stride bi * Si)
  int64_t d;               // plan dimension
  int64_t nsets;           // sets per row: (cols / d) * (d / (bo bi Si)) * Si
  int sets;                // sets per workgroup (at most 256 / (bo bi))
  int inner_first;         // inverse order
  int per_group;           // blocks per group (else one shared block per stage)
  const float* blk_o;      // outer stage blocks [group][j][k] (groups hi Si bi... as in the plan)
  const float* blk_i;
  int vec_i;               // blk_i 16-byte aligned and bi a multiple of 4: its rows load as float4
  const float* sign_in;    // applied at load (forward, first stage of the plan), or null
  const float* sign_out;   // applied at store (inverse, first stage of the plan), or null
  const void* src;
  int src_t;
  int64_t ld_src;
  void* dst;
  int dst_t;
  int64_t ld_dst;
  int64_t lines;           // rows, at most kP2MaxLines
};
// Set s (of the row) -> chunk c, hi, lo.
__host__ __device__ inline void p2_set(const P2Args& a, int64_t s, int64_t& c, int64_t& hi, int64_t& lo) {
  const int64_t per_chunk = a.d / (a.bo * a.bi * a.Si) * a.Si;
  c = s / per_chunk;
  const int64_t r = s - c * per_chunk;
  hi = r / a.Si;
  lo = r - hi * a.Si;
}
__host__ __device__ inline int64_t p2_pos(const P2Args& a, int64_t c, int64_t hi, int64_t lo, int ao, int bi_) {
  return c * a.d + hi * (a.bo * a.bi * a.Si) + (int64_t)ao * (a.bi * a.Si) + (int64_t)bi_ * a.Si + lo;
}
// Block row offsets: outer group hi (bi Si) + b Si + lo, inner group
// (hi bo + a) Si + lo (the stages' own group numbering within the chunk).
__host__ __device__ inline int64_t p2_row_o(const P2Args& a, int64_t hi, int64_t lo, int b, int j) {
  const int64_t g = a.per_group ? hi * (a.bi * a.Si) + (int64_t)b * a.Si + lo : 0;
  return (g * a.bo + j) * a.bo;
}
__host__ __device__ inline int64_t p2_row_i(const P2Args& a, int64_t hi, int64_t lo, int ao, int j) {
  const int64_t g = a.per_group ? (hi * a.bo + ao) * a.Si + lo : 0;
  return (g * a.bi + j) * a.bi;
}
__host__ __device__ inline int64_t p2_set_blocks(const P2Args& a) {
  return (a.nsets + a.sets - 1) / a.sets;
}
__host__ __device__ inline int64_t p2_blocks(const P2Args& a) {
  return p2_set_blocks(a) * ((a.lines + kP2Lines - 1) / kP2Lines);
}
// Workgroup blk -> set block sbk and rows kP2Lines * lb ..  Workgroups go to
// the XCDs in turn (blk mod 8); with the grid a multiple of 8, the workgroups
// of one XCD take consecutive (set block, line block) pairs, line blocks
// fastest, so the line blocks of a set and the block rows that neighbouring
// sets share in a cache line come into that XCD's L2 once.
__host__ __device__ inline void p2_tile(const P2Args& a, int64_t blk, int64_t& sbk, int64_t& lb) {
  const int64_t nb = p2_blocks(a), nlb = nb / p2_set_blocks(a);
  const int64_t lin = nb % 8 ? blk : (blk % 8) * (nb / 8) + blk / 8;
  sbk = lin / nlb;
  lb = lin % nlb;
}
hipError_t launch_stage_pair2(const P2Args& a, hipStream_t s);

// Stages [t_begin, t_end) of the plan only (t_end = -1: to the last), in
// forward order (inverse: the same range, transposed, last stage first); the
// signs go with stage 0, so a range that starts later applies none.
// nparts > 1 (right side, float32 x): x is nparts arrays part_stride elements
// apart whose sum is the input (SpArgs::nparts); only when the first launch
// is the tile kernel, else BRQ_ERR_UNSUPPORTED before anything is launched.
brq_status sp_rotate_stages(const Plan* p, int side, int inverse, int t_begin, int t_end,
                            const void* x, int xt, int64_t ldx, void* y, int yt, int64_t ldy,
                            int64_t rows, int64_t cols, void* ws, size_t ws_bytes, hipStream_t s,
                            hipError_t* herr, int nparts = 1, int64_t part_stride = 0);

}  // namespace brq
