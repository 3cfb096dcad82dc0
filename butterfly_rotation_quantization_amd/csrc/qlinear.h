// Quantized linear layer at decode: Z = X~ W'^T, the weight given as absmax
// codes and float32 scales (the output of rotate_quantize_pack).
//
// Dequantization happens in the product's prologue.  A b-bit code c stands
// for alpha (2c - L) / L with L = 2^b - 1, and 2c - L is an integer of at
// most 5 bits, exact in f16 and bf16; so the MFMA products (activation times
// integer) are exact, each quantizer group's partial sum is formed in
// float32 by v_mfma_f32_16x16x32_{f16,bf16}, and then scaled by alpha / L.
//
// A workgroup is four waves over 64 tn outputs (16 tn each) and 16 tm
// tokens: tm = 1, tn = 4 up to 16 tokens, tm = 4, tn = 2 above (the direct
// kernel), or tm = 1, tn = 2 (the streaming kernel).  Wave w owns
// outputs o0 + 16 tn w .. for all the tokens; it loads each activation
// operand once for its tn output tiles and decodes each weight code once for
// its tm token tiles.  Groups of 64 or 128 inputs.  The reduction over the
// input index is split into `splits` parts of kc (a multiple of the group)
// so that a few tokens still fill the GPU; the parts go to a float32 buffer
// [splits][T][m] and a second kernel sums them (in a fixed order).
//
// The index arithmetic lives here as __host__ __device__ functions so the
// host dry run checks exactly what the GPU executes.
#pragma once

#include "brq_internal.h"

namespace brq {

constexpr int kQlThreads = 256;
constexpr int kQlOut = 64;  // outputs per workgroup
constexpr int kQlTok = 16;  // tokens per workgroup

struct QlArgs {
  const void* x;        // X~ [T][ldx], f16 or bf16 (xt)
  int xt;
  int64_t ldx;
  int64_t T, m, n;
  const uint8_t* codes; // [m][codes_ld]: row o's codes, LSB-first
  const float* scales;  // [m][scales_ld] absmax alpha
  int bits, group;
  int64_t codes_ld, scales_ld;
  int splits;
  int64_t kc;           // input columns per split (a multiple of group)
  int tm;               // 16-token tiles per workgroup (1 or 4)
  int tn;               // 16-output tiles per wave
  int kind;             // QlKind
  int tv;               // kQlStream: LDS token rows of a tile (min(T, 16 tm))
  float* part;          // [splits][T][m]
};

// kQlDirect: every lane reads its codes and activations from global memory.
// kQlStream: one or two 16-token tiles per workgroup; the workgroup's weight rows
//   (codes and scales) and the tile's activations pass through LDS one chunk
//   of kQlChunk inputs at a time, with whole-line loads (each row's chunk is
//   contiguous, so every code byte leaves HBM once per token tile), and the
//   next chunk is loaded into registers while the current one is multiplied,
//   so the loads stay in flight during the arithmetic (no global load is
//   waited for inside it).  Several token tiles read the same weight block
//   one after another (the tiles of a row block are launched together, so
//   most re-reads hit the caches).  The decode work per code is the limit;
//   two tiles per workgroup (above 16 tokens, where the staging fits) halve
//   it per token, four tiles cost too many registers.
// kQlGemm (64 tokens and more): 128 tokens (eight 16-token tiles) x 256
//   weight rows per workgroup of eight waves, two per SIMD; wave w owns rows
//   32 w .. 32 w + 31 for all 128 tokens, so each code is decoded once for
//   128 tokens instead of 16 or 32.  Chunks of 256 inputs are staged in LDS
//   (codes, scales, activations) with the f16 activations already paired the
//   way the MFMA operands take them.  (tn = 4 keeps the row count per
//   workgroup as kQlOut tn.)  Workgroups are numbered so that the eight
//   (token tile, split) pairs of a weight row block go one to each XCD: an
//   XCD reads one slice of X~ from memory and serves it to every row block
//   from its L2.
enum QlKind { kQlDirect = 0, kQlStream = 1, kQlGemm = 2 };
constexpr int kQlStreamTn = 2;
constexpr int kQlGemmTm = 8;
constexpr int kQlGemmTn = 4;
constexpr int kQlGemmChunk = 256;
constexpr int kQlGemmMinT = 64;
constexpr int kQlGemmThreads = 512;  // eight waves
constexpr int kQlGemmTnw = 2;        // 16-row tiles per wave
constexpr int kQlGemmXcds = 8;  // (token tile, split) pairs per weight row block

struct QlTile {
  int64_t ct, tt, split;
};
// 16-output tiles per wave for a token tile count tm.
__host__ __device__ inline int ql_tn(int tm) { return tm == 4 ? 2 : 4; }
__host__ __device__ inline int64_t ql_ctiles(const QlArgs& a) { return a.m / (kQlOut * a.tn); }
__host__ __device__ inline int64_t ql_ttiles(const QlArgs& a) {
  return (a.T + kQlTok * a.tm - 1) / (kQlTok * a.tm);
}
__host__ __device__ inline int64_t ql_blocks(const QlArgs& a) {
  return ql_ctiles(a) * ql_ttiles(a) * a.splits;
}
// Output tiles run fastest: consecutive workgroups read consecutive weight rows.
// kQlGemm: the (token tile, split) pairs run fastest, so consecutive
// workgroups (which the dispatcher deals to the XCDs in turn) share a row
// block and each XCD keeps one (token tile, split) pair.
__host__ __device__ inline QlTile ql_tile(const QlArgs& a, int64_t bid) {
  QlTile t;
  const int64_t nc = ql_ctiles(a), nt = ql_ttiles(a);
  if (a.kind == kQlGemm) {
    const int64_t nts = nt * a.splits, r = bid % nts;
    t.ct = bid / nts;
    t.tt = r % nt;
    t.split = r / nt;
    return t;
  }
  t.ct = bid % nc;
  const int64_t r = bid / nc;
  t.tt = r % nt;
  t.split = r / nt;
  return t;
}
// Byte offset of the codes of row o, inputs k .. (k a multiple of 16).
__host__ __device__ inline int64_t ql_code_off(const QlArgs& a, int64_t o, int64_t k) {
  return o * a.codes_ld + k * a.bits / 8;
}
// The streaming kernel needs n a multiple of kQlChunk and 16-byte aligned codes.
constexpr int kQlChunk = 512;
// LDS row pitches for a chunk of ck inputs: the chunk's code bytes plus 16
// (keeps 16-byte alignment and moves successive rows by four banks); a
// token's activations plus 16.
__host__ __device__ constexpr int ql_code_pitch_ck(int bits, int ck) { return ck * bits / 8 + 16; }
__host__ __device__ constexpr int ql_xpitch(int ck) { return 2 * ck + 16; }
__host__ __device__ inline int ql_code_pitch(int bits) { return ql_code_pitch_ck(bits, kQlChunk); }
constexpr int kQlXPitch = ql_xpitch(kQlChunk);
// LDS of a staged launch: rows x (codes + scales of the chunk's groups), and
// tv activation rows.
__host__ __device__ inline size_t ql_lds_bytes_ck(int bits, int group, int rows, int tv, int ck) {
  return (size_t)rows * ql_code_pitch_ck(bits, ck) + (size_t)rows * (ck / group + 1) * 4 +
         (size_t)tv * ql_xpitch(ck);
}
__host__ __device__ inline size_t ql_lds_bytes(int bits, int group, int rows, int tv) {
  return ql_lds_bytes_ck(bits, group, rows, tv, kQlChunk);
}
// The LDS of a kQlGemm launch (at most 115 KiB, b <= 5); the launch takes
// all 128 token rows (rows past the last token hold zeros).
__host__ __device__ inline size_t ql_gemm_lds_bytes(int bits, int group, int tv) {
  return ql_lds_bytes_ck(bits, group, kQlOut * kQlGemmTn, tv, kQlGemmChunk);
}
// 16-token tiles per workgroup for T tokens.
__host__ __device__ inline int ql_tm(int64_t T) { return T > kQlTok ? 4 : 1; }
// The kernel for a shape (codes_aligned: 16-byte aligned codes): the GEMM-
// shaped kernel from 64 tokens when the rows come in blocks of 256 and the
// inputs in chunks of 256 (its launch opts in to up to 115 KiB of LDS); else
// the streaming kernel when its staging fits the 64 KiB a launch takes
// without an attribute (at most 62.75 KiB for b <= 5); else the direct one.
__host__ __device__ inline int ql_kind(int64_t T, int64_t m, int64_t n, int bits, int group, bool codes_aligned) {
  if (codes_aligned && T >= kQlGemmMinT && n % kQlGemmChunk == 0 && m % (kQlOut * kQlGemmTn) == 0)
    return kQlGemm;
  if (n % kQlChunk || !codes_aligned) return kQlDirect;
  if (ql_lds_bytes(bits, group, kQlOut * kQlStreamTn, (int)(T < kQlTok ? T : kQlTok)) <= 64 * 1024)
    return kQlStream;
  return kQlDirect;
}
// Token tiles per workgroup of the streaming kernel: two above 16 tokens when
// the staging of 32 activation rows still fits.
__host__ __device__ inline int ql_stream_tm(int64_t T, int bits, int group) {
  return T > kQlTok && ql_lds_bytes(bits, group, kQlOut * kQlStreamTn, (int)(T < 2 * kQlTok ? T : 2 * kQlTok)) <= 64 * 1024
             ? 2 : 1;
}
__host__ __device__ inline int ql_kind_tm(int kind, int64_t T, int bits, int group) {
  return kind == kQlGemm ? kQlGemmTm : kind == kQlStream ? ql_stream_tm(T, bits, group) : ql_tm(T);
}
__host__ __device__ inline int ql_kind_tn(int kind, int tm) {
  return kind == kQlGemm ? kQlGemmTn : kind == kQlStream ? kQlStreamTn : ql_tn(tm);
}
// Splits of a kQlGemm launch: one per XCD for each token tile (at least one),
// at most one per chunk of inputs.
__host__ __device__ inline int ql_gemm_splits(int64_t T, int64_t n) {
  const int64_t tt = (T + kQlTok * kQlGemmTm - 1) / (kQlTok * kQlGemmTm);
  int64_t s = tt >= kQlGemmXcds ? 1 : kQlGemmXcds / tt;
  if (s > n / kQlGemmChunk) s = n / kQlGemmChunk;
  return (int)(s < 1 ? 1 : s);
}

// kQlGemm staging.  Per chunk of CK inputs: R rows of codes (16-byte pieces)
// and scales (times 1/L), and the activations of up to 128 tokens in 16-byte
// pieces taken two at a time: the pieces whose inputs ql_group_tile's MFMA
// operands pair up are loaded by one thread and stored in operand order, so
// that each operand is one 16-byte LDS read.  A lane's NC inputs of a group
// form a block; within it, slot pair sp covers 16 inputs, stored as operand
// s2 = 0 then s2 = 1.  f16: operand s2 word i holds inputs (8 sp + 4 s2 + i',
// 8 sp + 4 s2 + i' + NC/2) for i' = 2i, 2i + 1 (as ql_group_tile's perms make
// them); bf16: inputs 16 sp .. 16 sp + 15 in order.
// Input offsets (within the chunk) of unit u's two natural pieces, and of
// its two stored operands (nc = G/4 inputs per lane block).
__host__ __device__ constexpr int ql_gemm_nat0(int u, int nc, bool bf) {
  return (u / (nc / 16)) * nc + (bf ? 16 : 8) * (u % (nc / 16));
}
__host__ __device__ constexpr int ql_gemm_nat1(int u, int nc, bool bf) { return ql_gemm_nat0(u, nc, bf) + (bf ? 8 : nc / 2); }
__host__ __device__ constexpr int ql_gemm_op0(int u, int nc) { return (u / (nc / 16)) * nc + 16 * (u % (nc / 16)); }
template <int BITS, int G, bool BF>
struct QlGemmPieces {
  static constexpr int R = kQlOut * kQlGemmTn, CK = kQlGemmChunk, NT = kQlGemmThreads;
  static constexpr int CB = CK * BITS / 8, NG = CK / G, NC = G / 4;
  static constexpr int UT = CK / 16;  // 16-input units per token
  static constexpr int NCP = R * (CB / 16) / NT, NSP = R * NG / NT;
  static constexpr int NXU = kQlTok * kQlGemmTm * UT / NT;  // units per thread
  static_assert(NCP * NT == R * (CB / 16) && NSP * NT == R * NG && NXU * NT == kQlTok * kQlGemmTm * UT,
                "staging pieces must divide among the threads");
  __host__ __device__ static constexpr int nat0(int u) { return ql_gemm_nat0(u, NC, BF); }
  __host__ __device__ static constexpr int nat1(int u) { return ql_gemm_nat1(u, NC, BF); }
  __host__ __device__ static constexpr int op0(int u) { return ql_gemm_op0(u, NC); }
};

hipError_t launch_qlinear(const QlArgs& a, hipStream_t s);
// Z[t][o] = sum over splits of part[s][t][o], into out (type ot, leading dimension ldo).
hipError_t launch_ql_reduce(const float* part, int splits, int64_t T, int64_t m, void* out, int ot,
                            int64_t ldo, hipStream_t s);

}  // namespace brq
