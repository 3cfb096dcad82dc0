// Host side of the stage pass (stage.h): which rotations take it, and the
// chain of one launch per stage.
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "stage.h"

namespace brq {

namespace {

// Largest line count (rows of a right-side rotation, columns of a left-side
// one) that takes the stage pass: below it the multi-stage tile pass leaves
// most of the GPU idle.
constexpr int64_t kSpMaxLines = 1024;

int pow2_at_least(int b) {
  int p = 1;
  while (p < b) p <<= 1;
  return p;
}

// The stages to run.  A Hadamard plan is the Sylvester matrix of order d
// whatever power-of-two radices it lists (H_{ab} = H_a (x) H_b in natural
// order, and the normalisations multiply to 1/sqrt(d)), so it runs as
// radix-16 stages plus one smaller remainder stage; other plans run as given.
struct StageList {
  int n = 0;
  int b[kMaxStages * 4];
  int64_t S[kMaxStages * 4];
  int t[kMaxStages * 4];  // plan stage (-1 for the canonical Hadamard stages)
};

StageList stages_of(const Plan* p) {
  StageList L;
  if (p->mode == BRQ_HADAMARD) {
    int rest = p->d;
    int64_t S = 1;
    int tmp_b[kMaxStages * 4];
    int64_t tmp_S[kMaxStages * 4];
    int k = 0;
    while (rest > 1) {  // from the stride-1 end
      const int b = rest >= 16 ? 16 : rest;
      tmp_b[k] = b;
      tmp_S[k] = S;
      S *= b;
      rest /= b;
      ++k;
    }
    for (int i = 0; i < k; ++i) {  // stage 0 is the most significant digit
      L.b[i] = tmp_b[k - 1 - i];
      L.S[i] = tmp_S[k - 1 - i];
      L.t[i] = -1;
    }
    L.n = k;
    return L;
  }
  for (int i = 0; i < p->nst; ++i) {
    L.b[i] = p->radix[i];
    L.S[i] = p->stride[i];
    L.t[i] = i;
  }
  L.n = p->nst;
  return L;
}

}  // namespace

bool sp_shape_ok(const Plan* p, int side, int64_t rows, int64_t cols) {
  if (!p || rows <= 0 || cols <= 0) return false;
  const int64_t lines = side == 0 ? rows : cols;
  const int64_t axis = side == 0 ? cols : rows;  // positions fit sp_pos's 32 bits
  if (axis % p->d || axis > (int64_t)1 << 30) return false;
  // grid: line tiles of the size the launch will use times at most axis / 2 group tiles
  const int64_t tl = side != 0 ? kSpLines : (lines <= kSpTinyRows ? kSpLinesTiny : kSpLinesFew);
  if (((lines + tl - 1) / tl) * (axis / 2) >= ((int64_t)1 << 31)) return false;
  for (int i = 0; i < p->nst; ++i)
    if (p->radix[i] > 64) return false;
  return true;
}

bool sr_supported(const SpArgs& a) {
  if (a.side != 1 || a.b2 || a.b < 2 || a.b > 64 || (a.b & (a.b - 1))) return false;
  if (a.mode == BRQ_HADAMARD ? a.b > 16 : !a.blk) return false;
  if (a.src_t != BRQ_F32 && a.dst_t != BRQ_F32) return false;
  if (a.ngroups != a.ngc || a.d >= ((int64_t)1 << 31)) return false;  // one chunk: the rows
  const int vec = sr_vec(a.b);
  const int in_bytes = a.src_t == BRQ_F32 ? 4 : 2, out_bytes = a.dst_t == BRQ_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(a.src) % (vec * in_bytes) ||
      reinterpret_cast<uintptr_t>(a.dst) % (vec * out_bytes) || a.ld_src % vec || a.ld_dst % vec || a.lines % vec)
    return false;
  return sr_col_tiles(a) * a.ngroups < ((int64_t)1 << 31);
}

bool sl_supported(const SpArgs& a) {
  // up to 32 rows the tile kernel's 8-row tiles spread wider and are faster
  // (measured 30.6 against 32.6 us on the 70B decode at 16 rows)
  if (a.side != 0 || a.b2 || a.b < 2 || (a.b > 8 && a.b != 16) || a.S % kSlLanes ||
      a.ngroups % kSlLanes || a.lines <= 32)
    return false;
  if (a.mode != BRQ_HADAMARD && !a.blk) return false;
  if (a.b == 16 && a.mode != BRQ_HADAMARD && !a.blk_vec) return false;  // float4 block rows
  // radix 16: each workgroup reads its 64 blocks (64 KB), which pays off for
  // a few rows (latency) or many (the blocks amortised over 32 rows and more);
  // in between the tile kernel moves less (measured: 31 vs 44 us at 256 rows)
  if (a.b == 16 && a.lines > 32 && a.lines < 4096) return false;
  const SlGeom g = sl_geom(a, sl_rows_per(a));
  return g.lo_tiles * g.row_tiles < ((int64_t)1 << 31);
}

// Rows per workgroup: as many as keep at least 2048 workgroups, at most 64
// (radix <= 8: the four waves take every fourth row, so a multiple of 4).
int sl_rows_per(const SpArgs& a) {
  const int64_t lo_tiles = a.ngroups / kSlLanes;
  const int minr = a.b == 16 ? 1 : 4;
  int r = 64;
  while (r > minr && lo_tiles * ((a.lines + r - 1) / r) < 2048) r /= 2;
  return r;
}

bool sp_rotate_supported(const Plan* p, int side, int64_t rows, int64_t cols) {
  if (!sp_shape_ok(p, side, rows, cols)) return false;
  // dense blocks: a block row in registers beats the tile pass's per-output
  // block reads at any size; Hadamard plans only where the tile pass starves
  return p->mode != BRQ_HADAMARD || (side == 0 ? rows : cols) <= kSpMaxLines;
}

brq_status sp_rotate(const Plan* p, int side, int inverse, const void* x, int xt, int64_t ldx,
                     void* y, int yt, int64_t ldy, int64_t rows, int64_t cols, void* ws,
                     size_t ws_bytes, hipStream_t s, hipError_t* herr) {
  return sp_rotate_stages(p, side, inverse, 0, -1, x, xt, ldx, y, yt, ldy, rows, cols, ws,
                          ws_bytes, s, herr);
}

brq_status sp_rotate_stages(const Plan* p, int side, int inverse, int t_begin, int t_end,
                            const void* x, int xt, int64_t ldx, void* y, int yt, int64_t ldy,
                            int64_t rows, int64_t cols, void* ws, size_t ws_bytes, hipStream_t s,
                            hipError_t* herr, int nparts, int64_t part_stride) {
  *herr = hipSuccess;
  const bool parts = nparts > 1;
  if (parts && (side != 0 || xt != BRQ_F32 || part_stride < rows * ldx)) return BRQ_ERR_UNSUPPORTED;
  StageList L = stages_of(p);
  if (t_end < 0) t_end = L.n;
  if (t_begin < 0 || t_end > L.n || t_begin >= t_end) return BRQ_ERR_UNSUPPORTED;
  const bool signs_here = t_begin == 0;  // the signs go with stage 0
  {  // keep stages [t_begin, t_end) of the list
    StageList R;
    for (int i = t_begin; i < t_end; ++i) {
      R.b[R.n] = L.b[i];
      R.S[R.n] = L.S[i];
      R.t[R.n] = L.t[i];
      ++R.n;
    }
    L = R;
  }
  // intermediate: y itself when it is float32, else the workspace
  void* mid = y;
  int64_t ldm = ldy;
  if (L.n > 1 && yt != BRQ_F32) {
    if (!ws || ws_bytes < (size_t)rows * cols * sizeof(float)) return BRQ_ERR_WORKSPACE;
    mid = ws;
    ldm = cols;
  }
  const int64_t lines = side == 0 ? rows : cols;
  for (int i = 0; i < L.n; ++i) {
    const int si = inverse ? L.n - 1 - i : i;
    // two consecutive right-side stages of radix <= 16 (product <= 256) for
    // up to 32 rows: one launch (a trailing forward or leading inverse (16, 16)
    // at strides 16 and 1 keeps its own pair kernel)
    if (side == 0 && lines <= kP2MaxLines && p->mode != BRQ_HADAMARD && i + 1 < L.n) {
      const int sn = inverse ? si - 1 : si + 1;
      const int to = si < sn ? si : sn, ti = si < sn ? sn : si;  // outer (larger stride), inner
      const bool pair16 = L.b[to] == 16 && L.b[ti] == 16 && L.S[to] == 16 && L.S[ti] == 1;
      if (!pair16 && L.b[to] <= 16 && L.b[ti] <= 16 && L.b[to] * L.b[ti] <= 256) {
        if (parts && i == 0) return BRQ_ERR_UNSUPPORTED;  // the pair kernel reads one array
        P2Args q;
        std::memset(&q, 0, sizeof q);
        q.bo = L.b[to];
        q.bi = L.b[ti];
        q.Si = L.S[ti];
        q.d = p->d;
        q.nsets = (cols / p->d) * (p->d / (q.bo * q.bi * q.Si)) * q.Si;
        q.sets = 256 / (q.bo * q.bi);
        // fewer workgroups than compute units: one set per workgroup
        if (p2_blocks(q) < 256) q.sets = 1;
        q.inner_first = inverse ? 1 : 0;
        q.per_group = p->mode == BRQ_PER_GROUP ? 1 : 0;
        const float* base = inverse ? p->blkT : p->blk;
        q.blk_o = base + p->blk_off[L.t[to]];
        q.blk_i = base + p->blk_off[L.t[ti]];
        q.vec_i = q.bi % 4 == 0 && reinterpret_cast<uintptr_t>(q.blk_i) % 16 == 0 ? 1 : 0;
        const bool last = i + 1 == L.n - 1;
        q.sign_in = (!inverse && i == 0 && signs_here) ? p->signs : nullptr;
        q.sign_out = (inverse && last && signs_here) ? p->signs : nullptr;
        q.src = i == 0 ? x : mid;
        q.src_t = i == 0 ? xt : BRQ_F32;
        q.ld_src = i == 0 ? ldx : ldm;
        q.dst = last ? y : mid;
        q.dst_t = last ? yt : BRQ_F32;
        q.ld_dst = last ? ldy : ldm;
        q.lines = lines;
        if (p2_blocks(q) >= ((int64_t)1 << 31)) return BRQ_ERR_UNSUPPORTED;
        char name[64];
        snprintf(name, sizeof name, "stage R%s(%d,%d) S%lld", inverse ? "^T" : "", L.b[si], L.b[sn],
                 (long long)L.S[si]);
        const int tok = prof_begin(name, s);
        const hipError_t e = launch_stage_pair2(q, s);
        prof_end(tok, s);
        if (e != hipSuccess) {
          *herr = e;
          return BRQ_ERR_HIP;
        }
        ++i;
        continue;
      }
    }
    SpArgs a;
    std::memset(&a, 0, sizeof a);
    a.side = side;
    // right side: 8-row tiles (measured faster than 32-row ones from 1 row
    // to 8192: more workgroups, fewer registers and less LDS each), 4-row
    // tiles up to 16 rows (the decode rotations at 16 tokens: the (16, 16)
    // pair 10.8 -> 9.8 us, the decode linear's output rotation 22 -> 17 us;
    // at 256 rows 4-row tiles were slower)
    a.tile_lines = side == 0 ? (lines <= kSpTinyRows ? kSpLinesTiny : kSpLinesFew) : 0;
    a.b = L.b[si];
    a.bp = pow2_at_least(a.b);
    a.bs = (a.b + 3) & ~3;
    a.gw = kSpThreads / a.bp;
    if (a.gw * a.bs > kSpLineFloats) a.gw = kSpLineFloats / a.bs;
    // a right-side pair runs in one launch, the tile one block of 256
    // consecutive positions: forward (16, S = 16) then (16, 1), inverse
    // (16, 1) then (16, S = 16) (the transposed blocks)
    const int sn = inverse ? si - 1 : si + 1;  // the next stage
    const float* base = inverse ? p->blkT : p->blk;
    const bool pair = side == 0 && i + 1 < L.n && L.b[si] == 16 && L.b[sn] == 16 &&
                      L.S[si] == (inverse ? 1 : 16) && L.S[sn] == (inverse ? 16 : 1) &&
                      (p->mode == BRQ_HADAMARD || reinterpret_cast<uintptr_t>(base + p->blk_off[L.t[sn]]) % 16 == 0);
    if (pair) {
      a.gw = 16;
      a.b2 = L.b[sn];
      a.inv2 = inverse ? 1 : 0;
      a.blk2 = p->mode == BRQ_HADAMARD ? nullptr : base + p->blk_off[L.t[sn]];
    }
    a.mode = p->mode;
    a.S = L.S[si];
    a.d = p->d;
    a.ngc = p->d / a.b;
    a.ngroups = (side == 0 ? cols / p->d : 1) * a.ngc;
    a.lines = lines;
    a.hscale = 1.0f / std::sqrt((float)a.b);
    a.blk = p->mode == BRQ_HADAMARD
                ? nullptr
                : (inverse ? p->blkT : p->blk) + p->blk_off[L.t[si]];
    a.blk_vec = a.blk && a.b % 4 == 0 && reinterpret_cast<uintptr_t>(a.blk) % 16 == 0;
    a.sign_in = (!inverse && i == 0 && signs_here) ? p->signs : nullptr;
    a.sign_out = (inverse && i + (pair ? 1 : 0) == L.n - 1 && signs_here) ? p->signs : nullptr;
    a.src = i == 0 ? x : mid;
    a.src_t = i == 0 ? xt : BRQ_F32;
    a.ld_src = i == 0 ? ldx : ldm;
    const bool last = i + (pair ? 1 : 0) == L.n - 1;
    a.dst = last ? y : mid;
    a.dst_t = last ? yt : BRQ_F32;
    a.ld_dst = last ? ldy : ldm;
    if (parts && i == 0) {
      a.nparts = nparts;
      a.part_stride = part_stride;
    }
    const bool rows_kernel = !a.nparts && sr_supported(a);
    const bool lanes_kernel = !a.nparts && !rows_kernel && sl_supported(a);
    if (parts && i == 0 && (rows_kernel || lanes_kernel)) return BRQ_ERR_UNSUPPORTED;
    if (!rows_kernel && !lanes_kernel && sp_blocks(a) >= ((int64_t)1 << 31)) return BRQ_ERR_UNSUPPORTED;  // grid
    char name[64];
    if (pair)
      snprintf(name, sizeof name, "stage R%s(%d,%d) S%lld", inverse ? "^T" : "", a.b, a.b2, (long long)a.S);
    else
      snprintf(name, sizeof name, "stage %s%s(%d) S%lld", side == 0 ? "R" : "L",
               inverse ? "^T" : "", a.b, (long long)a.S);
    const int tok = prof_begin(name, s);
    const hipError_t e = rows_kernel    ? launch_stage_rows(a, s)
                         : lanes_kernel ? launch_stage_lanes(a, sl_rows_per(a), s)
                                        : launch_stage(a, s);
    prof_end(tok, s);
    if (e != hipSuccess) {
      *herr = e;
      return BRQ_ERR_HIP;
    }
    if (pair) ++i;  // the second stage of the pair is done
  }
  return BRQ_OK;
}

}  // namespace brq
