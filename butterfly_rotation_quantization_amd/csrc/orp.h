// ORP GEO quantizer: launch arguments and the index arithmetic shared by the
// kernels (orp.hip) and the host dry-run checker.
//
// [ORPQuant] technical summary, section 2: per vector w (here a contiguous
// group of `group` inputs of one row), a primary basis b1 on an asymmetric
// power-of-two lattice with zero, a secondary basis b2 orthogonal to it made
// by exchanging entries at stride S inside micro-blocks of 2S and flipping
// signs, and the least-squares scales c_i = <w, b_i> / ||b_i||^2 (GEO mode).
//
// Geometry: one wavefront takes kOrpChunk consecutive elements of one row,
// kOrpPerLane per lane; a group of g elements spans g / kOrpPerLane lanes.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kOrpThreads = 256;  // four wavefronts per workgroup
constexpr int kOrpPerLane = 8;
constexpr int kOrpChunk = 64 * kOrpPerLane;
constexpr int kOrpChunksPerWave = 4;  // consecutive chunks, all loads issued first

struct OrpArgs {
  // quantize input
  const void* w;
  int wt;
  int64_t ldw;
  const float* smooth;  // per-input-channel preconditioning [n], or nullptr
  // shape and quantizer
  int64_t m, n;
  int bits, group, stride;
  int64_t chunks;       // kOrpChunk-element chunks per row: ceil(n / kOrpChunk)
  int lg_group, lg_stride;  // log2 of group and stride
  int64_t codes_ld, signs_ld, coef_ld;  // per row: n*bits/8 bytes, n/16 bytes, 2*n/group floats
  // quantize outputs / dequant inputs
  uint8_t* codes;       // [m][n*bits/8]
  uint8_t* signs;       // [m][n/16]: one bit per pair
  float* coef;          // [m][n/group][2]: (c1, c2)
  // dequant output
  void* out;
  int ot;
  int64_t ldo;
};

// Pair number of the pair whose first entry is i (i in the first half of its
// micro-block of 2S): pairs are numbered in the order of their first entries.
__host__ __device__ inline int64_t orp_pair(int64_t i, int S) {
  return (i / (2 * S)) * S + (i % (2 * S));
}
// The same for S = 2^lg (32-bit column indices).
__host__ __device__ inline uint32_t orp_pair_lg(uint32_t i, int lg) {
  return ((i >> (lg + 1)) << lg) + (i & ((2u << lg) - 1));
}

// Chunk ci (0 <= ci < m * chunks, row-major): its row and first column.
// Wavefront w takes chunks w * kOrpChunksPerWave .. + kOrpChunksPerWave - 1.
__host__ __device__ inline void orp_chunk(const OrpArgs& a, int64_t ci, int64_t* row, int64_t* c0) {
  *row = ci / a.chunks;
  *c0 = (ci - *row * a.chunks) * kOrpChunk;
}

__host__ __device__ inline int64_t orp_total_chunks(const OrpArgs& a) { return a.m * a.chunks; }
inline int64_t orp_waves(const OrpArgs& a) {
  return (orp_total_chunks(a) + kOrpChunksPerWave - 1) / kOrpChunksPerWave;
}
inline int64_t orp_blocks(const OrpArgs& a) {
  return (orp_waves(a) + kOrpThreads / 64 - 1) / (kOrpThreads / 64);
}

hipError_t launch_orp_quant(const OrpArgs& a, hipStream_t s);
hipError_t launch_orp_dequant(const OrpArgs& a, hipStream_t s);

}  // namespace brq
