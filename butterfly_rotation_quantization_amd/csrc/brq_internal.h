// Internal types shared by the host layer and the kernels of libbrq.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "brq.h"

namespace brq {

constexpr int kMaxStages = 16;     // stages per plan
constexpr int kMaxPassStages = 16; // stages of one side inside one pass
constexpr int kMaxLevels = 32;     // codebook entries (5 bits)

// Device copy of a plan plus host metadata.
struct Plan {
  int device = -1;
  int d = 0;
  int nst = 0;
  int mode = BRQ_HADAMARD;
  int radix[kMaxStages] = {};
  int stride[kMaxStages] = {};       // S_t = prod_{s>t} b_s
  size_t blk_off[kMaxStages] = {};   // float offset of stage t in the block arrays
  float* blk = nullptr;              // blocks as given, [group][j][k] (or [j][k] shared)
  float* blkT = nullptr;             // the same blocks transposed, for the inverse
  float* signs = nullptr;            // +-1 as float, or nullptr
  float* signs_s = nullptr;          // Hadamard plans: the signs times 1 / sqrt(d)
  // Fast-path data (fused_prepare), for plans whose stage 0 has radix
  // <= 64 and whose last two stages are radix 16 (Hadamard plans as
  // (d / 256, 16, 16)): stage-0 blocks with the signs folded in, zero-padded
  // to 16*fz_nb and split into f16 (bh, bl) entries: as pass A's U_0 (fz0u,
  // radix 16 or 32 only) and in pass A's V_0 fragment order (fz0v); halves
  // between groups (0 = one block shared by all groups).
  int fz_ok = 0;
  int fz_b0 = 0;                     // radix of the fast path's stage 0
  int fz_s0 = 0;                     // its stride (d / fz_b0; 256 for Hadamard plans)
  int fz_nb = 0;
  uint16_t* fz0u = nullptr;
  uint16_t* fz0v = nullptr;
  int64_t fz_gs0u = 0, fz_gs0v = 0;
  int64_t fz_n0u = 0, fz_n0v = 0;    // extents in halves
  int fz0_exact = 0;                 // every stage-0 entry exact in f16
  // Pass B's blocks (the last two stages when both are radix 16) split into
  // f16 pairs, laid out as fused.h describes: stage nst-2 first, stage nst-1
  // at fzh_off2 halves; fzh_gs halves between groups (0 = shared).  Only
  // set when every block row has norm at most 1 + 1e-3.
  uint16_t* fzh = nullptr;
  int64_t fzh_off2 = 0;
  int64_t fzh_gs = 0;
  int64_t fzh_n = 0;                 // halves per stage
  int fzh_exact = 0;                 // every entry exact in f16
};

// One stage applied inside a pass, along one axis of the tile.
struct StageDesc {
  int b;            // radix
  int ls;           // local stride in tile k-units: S_t / S_pass
  int St;           // global stride S_t
  int mode;         // brq_block_mode
  const float* blk; // forward blocks (or transposed ones for the inverse)
};

// One axis of a 2-D tile.  Element e of the axis (0 <= e < P*W) has k = e / W,
// w = e % W and sits at index chunk*d + hi*P*S + k*S + lo0 + w.
struct AxisDesc {
  int P, S, W;        // tile extent P*W
  int d;              // length of one chunk along the axis
  int nhi, nlo;       // tiles along the axis within one chunk: d/(P*S), S/W
  int nchunk;         // chunks (block-diagonal right side); 1 otherwise
  int64_t D;          // full extent (rows or cols of the matrix)
  int ragged;         // stage-free axis whose last tile may be partial
  int nst;            // stages of this axis in the pass
  StageDesc st[kMaxPassStages];
  const float* sign;  // signs of this axis' side: applied at load (forward) / store (inverse)
  int sign_mod;       // length of that side's sign vector (index = position mod sign_mod)
};

enum Prologue { PRO_LOAD = 0, PRO_DEQUANT = 1 };
enum Epilogue { EPI_STORE = 0, EPI_QUANT = 1 };

struct PassArgs {
  AxisDesc ax[2];          // 0: row axis (left-side stages), 1: column axis (right side)
  int64_t m, n;            // matrix shape
  const void* src;         // PRO_LOAD source
  int src_t;
  int64_t ld_src;
  void* dst;               // EPI_STORE destination
  int dst_t;
  int64_t ld_dst;
  int inverse;
  int pro, epi;
  // quantizer (both the epilogue and the dequant prologue)
  int qkind, bits, group, nlev;
  float h;                 // (2^bits - 1)/2
  float sqrt_g;            // sqrt(group) in float32
  float cent[kMaxLevels];  // codebook centroids
  float tau[kMaxLevels];   // codebook thresholds (midpoints, float32)
  uint8_t* codes;          // quant output [m][n*bits/8]
  void* scales;            // quant output [m][n/group]
  const uint8_t* in_codes; // dequant input
  const void* in_scales;
  int64_t codes_ld;        // bytes per code row = n*bits/8
  int64_t scales_ld;       // scales per row = n/group
};

// Launch one generic pass over all tiles (pass_kernel.hip; the host dry-run
// build replaces it with a walk of every index the kernel would touch).
hipError_t launch_pass(const PassArgs& a, hipStream_t s);

// Device runtime used by the host layer (runtime.cpp; host memory in the
// dry-run build).
hipError_t rt_get_device(int* dev);
hipError_t rt_malloc(void** p, size_t bytes);
hipError_t rt_copy_to_device(void* dst, const void* src, size_t bytes);
hipError_t rt_copy_to_host(void* dst, const void* src, size_t bytes);
hipError_t rt_cu_count(int dev, int* cus);
void rt_free(void* p);

// Set this thread's brq_last_error text and return `s` (for entry points
// defined outside the host layer's file).
brq_status report_error(brq_status s, const char* msg);

// Kernel timing (brq_profile_*): bracket a launch with events on its stream
// when profiling is enabled; both calls are no-ops otherwise.
int prof_begin(const char* name, hipStream_t s);
void prof_end(int token, hipStream_t s);

// ---- index arithmetic of a tile pass, shared by the kernel and the host
// dry-run checker (one definition, so the checker tests what the GPU runs).

// Number of tiles of a pass along an axis.
__host__ __device__ inline int64_t axis_tiles(const AxisDesc& x) {
  if (x.ragged) return (x.D + x.P - 1) / x.P;
  return (int64_t)x.nchunk * x.nhi * x.nlo;
}

// Position of a tile along one axis.
struct AxisPos {
  int64_t base;     // global index of element (k=0, w=0)
  int64_t relbase;  // the same, relative to the start of its chunk
  int64_t limit;    // number of valid elements in this tile along the axis
};

__host__ __device__ inline AxisPos axis_pos(const AxisDesc& x, int64_t tile) {
  AxisPos p;
  if (x.ragged) {
    p.base = tile * x.P;
    p.relbase = p.base;
    const int64_t rem = x.D - p.base;
    p.limit = rem < x.P ? rem : x.P;
    return p;
  }
  const int64_t per_chunk = (int64_t)x.nhi * x.nlo;
  const int64_t chunk = tile / per_chunk;
  const int64_t r = tile - chunk * per_chunk;
  const int64_t hi = r / x.nlo;
  const int64_t lo0 = (r - hi * x.nlo) * x.W;
  p.relbase = hi * x.P * x.S + lo0;
  p.base = chunk * x.d + p.relbase;
  p.limit = (int64_t)x.P * x.W;
  return p;
}

// Offset of tile element e (0 <= e < P*W) from the tile base.
__host__ __device__ inline int64_t axis_off(const AxisDesc& x, int e) {
  if (x.ragged) return e;
  const int k = e / x.W;
  const int w = e - k * x.W;
  return (int64_t)k * x.S + w;
}

// Group `gid` of a stage inside a tile: members j = 0..b-1 sit at tile
// elements e0 + j*estep; k0/w locate member 0.
struct TileGroup {
  int k0, w, e0, estep;
};

__host__ __device__ inline TileGroup tile_group(const StageDesc& st, const AxisDesc& ax, int gid) {
  TileGroup g;
  g.w = gid % ax.W;
  const int q = gid / ax.W;
  const int kl = q % st.ls;
  const int kh = q / st.ls;
  g.k0 = kh * st.b * st.ls + kl;
  g.e0 = g.k0 * ax.W + g.w;
  g.estep = st.ls * ax.W;
  return g;
}

// Global group index c = (i / (b*S_t))*S_t + i % S_t of the group whose
// member 0 has chunk-relative index i.
__host__ __device__ inline int64_t group_index(const StageDesc& st, const AxisDesc& ax,
                                               int64_t relbase, const TileGroup& g) {
  const int64_t i0 = relbase + (int64_t)g.k0 * ax.S + g.w;
  const int64_t span = (int64_t)st.b * st.St;
  return (i0 / span) * st.St + (i0 % st.St);
}

}  // namespace brq
