// C ABI of libbrq: argument validation, plans, pass planning and dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "brq_internal.h"
#include "fused.h"
#include "rowhad.h"
#include "harp.h"
#include "orp.h"
#include "qlinear.h"
#include "stage.h"

struct brq_plan {
  brq::Plan p;
  std::vector<int8_t> signs;  // host copy of the signs (empty: all +1)
  // plans made from HARP parameters keep them, so they serialise compactly
  bool harp = false;
  std::vector<int8_t> theta;
  std::vector<float> scales, bases;
};

namespace brq {
namespace {

thread_local std::string g_last_error;

brq_status fail(brq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

brq_status hip_fail(hipError_t e, const char* what) {
  return fail(BRQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

brq_status report_error(brq_status s, const char* msg) { return fail(s, "%s", msg); }

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

std::atomic<int> g_path{BRQ_PATH_AUTO};
bool fast_paths() { return g_path.load(std::memory_order_relaxed) == BRQ_PATH_AUTO; }

bool valid_dtype(int32_t t) { return t == BRQ_F32 || t == BRQ_BF16 || t == BRQ_F16; }

// Tile budget of the generic pass (float32 elements held in LDS).
constexpr int kTileFloats = 16384;
constexpr int kMaxGroupP = 4096;

// A run of consecutive stages [a, e] of one side, executed in one pass.
struct Group {
  int a, e;
  int P, S;
};

std::vector<Group> side_groups(const Plan& p) {
  std::vector<Group> out;
  int e = p.nst - 1;
  while (e >= 0) {
    int a = e;
    int P = p.radix[e];
    while (a > 0 && (int64_t)P * p.radix[a - 1] <= kMaxGroupP &&
           e - (a - 1) + 1 <= kMaxPassStages) {
      --a;
      P *= p.radix[a];
    }
    out.push_back(Group{a, e, P, p.stride[e]});
    e = a - 1;
  }
  std::reverse(out.begin(), out.end());  // forward order: the group holding stage 0 first
  return out;
}

int largest_divisor_at_most(int s, int cap) {
  for (int w = std::min(s, cap); w >= 1; --w)
    if (s % w == 0) return w;
  return 1;
}

// Axis that carries the stages of `g` of plan `p`.
void stage_axis(AxisDesc& x, const Plan& p, const Group& g, int64_t D, bool inverse,
                int line_budget_floats) {
  std::memset(&x, 0, sizeof x);
  x.P = g.P;
  x.S = g.S;
  int W = largest_divisor_at_most(g.S, 16);
  while (W > 1 && (int64_t)g.P * W > line_budget_floats) {
    W = largest_divisor_at_most(g.S, W - 1);
  }
  x.W = W;
  x.d = p.d;
  x.nhi = p.d / (g.P * g.S);
  x.nlo = g.S / W;
  x.nchunk = (int)(D / p.d);
  x.D = D;
  x.ragged = 0;
  x.nst = g.e - g.a + 1;
  for (int i = 0; i < x.nst; ++i) {
    const int t = inverse ? (g.e - i) : (g.a + i);
    StageDesc& s = x.st[i];
    s.b = p.radix[t];
    s.St = p.stride[t];
    s.ls = p.stride[t] / g.S;
    s.mode = p.mode;
    s.blk = p.mode == BRQ_HADAMARD ? nullptr : ((inverse ? p.blkT : p.blk) + p.blk_off[t]);
  }
}

void free_axis(AxisDesc& x, int64_t D, int extent) {
  std::memset(&x, 0, sizeof x);
  x.P = extent;
  x.S = 1;
  x.W = 1;
  x.d = (int)std::min<int64_t>(D, 1 << 30);
  x.nhi = 1;
  x.nlo = 1;
  x.nchunk = 1;
  x.D = D;
  x.ragged = 1;
}

int lines_for(int64_t tile_line_floats) {
  int64_t L = kTileFloats / std::max<int64_t>(tile_line_floats, 1);
  if (L > 16) L = 16;
  if (L < 1) L = 1;
  return (int)L;
}

// Host check of everything the kernel's index arithmetic relies on; a pass
// that fails it is never launched.
const char* check_axis(const AxisDesc& x) {
  if (x.P < 1 || x.W < 1 || x.S < 1) return "axis extent";
  if (x.nst < 0 || x.nst > kMaxPassStages) return "stage count";
  if (x.ragged) {
    if (x.nst) return "stages on a ragged axis";
    if (x.W != 1 || x.S != 1) return "ragged axis layout";
    return nullptr;
  }
  if (x.S % x.W || x.nlo * x.W != x.S) return "lo tiling";
  if ((int64_t)x.P * x.S * x.nhi != x.d) return "hi tiling";
  if ((int64_t)x.nchunk * x.d != x.D) return "chunk tiling";
  int64_t span = 1;
  for (int i = 0; i < x.nst; ++i) {
    const StageDesc& s = x.st[i];
    if (s.b < 2 || s.b > 64) return "radix";
    if (s.ls < 1 || (int64_t)s.ls * x.S != s.St) return "local stride";
    if (x.P % ((int64_t)s.ls * s.b)) return "stage digit outside the pass";
    if (x.d % ((int64_t)s.b * s.St)) return "stage stride";
    if (s.mode != BRQ_HADAMARD && !s.blk) return "missing blocks";
    span *= s.b;
  }
  if (x.nst && span != x.P) return "pass extent != product of its radices";
  if (x.sign && x.sign_mod < 1) return "sign length";
  return nullptr;
}

const char* check_pass(const PassArgs& a) {
  for (int i = 0; i < 2; ++i)
    if (const char* why = check_axis(a.ax[i])) return why;
  if (!a.ax[0].ragged && a.ax[0].D != a.m) return "row axis extent";
  if (!a.ax[1].ragged && a.ax[1].D != a.n) return "column axis extent";
  if (a.ax[0].ragged && a.ax[0].D != a.m) return "row axis extent";
  if (a.ax[1].ragged && a.ax[1].D != a.n) return "column axis extent";
  const int64_t RT = (int64_t)a.ax[0].P * a.ax[0].W;
  const int64_t CT = (int64_t)a.ax[1].P * a.ax[1].W;
  if (RT * (CT + 1) * 4 > 96 * 1024) return "tile exceeds LDS";
  if (a.pro == PRO_LOAD && !a.src) return "source";
  if (a.pro == PRO_DEQUANT && (!a.in_codes || !a.in_scales)) return "dequant inputs";
  if (a.epi == EPI_STORE && !a.dst) return "destination";
  if (a.epi == EPI_QUANT) {
    if (!a.codes || !a.scales) return "quant outputs";
    if (a.group < 64 || a.group > 1024 || CT % a.group) return "quant group vs tile";
    const AxisDesc& c = a.ax[1];
    if (!c.ragged && !(c.S == 1 && c.W == 1)) return "quant tile columns not contiguous";
    if (c.ragged && c.P % a.group) return "quant tile columns";
  }
  if (a.pro == PRO_DEQUANT || a.epi == EPI_QUANT) {
    if (a.nlev != (1 << a.bits) || a.nlev > kMaxLevels) return "levels";
    if (a.codes_ld * 8 != a.n * a.bits || a.scales_ld * a.group != a.n) return "code layout";
  }
  return nullptr;
}

// Kernel name for timing: the stages the pass applies and its prologue/epilogue.
std::string pass_name(const PassArgs& a) {
  std::string n = "pass";
  if (a.pro == PRO_DEQUANT) n += " dequant";
  const char* side[2] = {" L", " R"};
  for (int i = 0; i < 2; ++i) {
    const AxisDesc& x = a.ax[i];
    if (!x.nst) continue;
    n += side[i];
    n += a.inverse ? "^T(" : "(";
    for (int t = 0; t < x.nst; ++t) {
      if (t) n += ",";
      n += std::to_string(x.st[t].b);
    }
    n += ")";
  }
  if (a.epi == EPI_QUANT) n += " quant";
  return n;
}

hipError_t checked_launch(const PassArgs& a, hipStream_t s, brq_status* st) {
  if (const char* why = check_pass(a)) {
    *st = fail(BRQ_ERR_UNSUPPORTED, "internal pass check failed: %s", why);
    return hipErrorInvalidValue;
  }
  const int tok = prof_begin(pass_name(a).c_str(), s);
  hipError_t e = launch_pass(a, s);
  prof_end(tok, s);
  *st = e == hipSuccess ? BRQ_OK : hip_fail(e, "pass launch");
  return e;
}

// The pass list of a transform.  Forward: the left side's groups, then the
// right side's (the sides commute).  Inverse: the reverse, each group's
// stages reversed with transposed blocks.
struct PassSpec {
  bool has_u, has_v;
  Group gu, gv;
};

std::vector<PassSpec> plan_passes(const Plan* U, const Plan* V) {
  std::vector<PassSpec> out;
  if (U)
    for (const Group& g : side_groups(*U)) out.push_back(PassSpec{true, false, g, Group{}});
  if (V)
    for (const Group& g : side_groups(*V)) out.push_back(PassSpec{false, true, Group{}, g});
  return out;
}

void build_axes(PassArgs& a, const PassSpec& ps, const Plan* U, const Plan* V, int64_t m,
                int64_t n, bool inverse) {
  if (ps.has_u) {
    stage_axis(a.ax[0], *U, ps.gu, m, inverse, kTileFloats / 16);
    const int line = a.ax[0].P * a.ax[0].W;
    free_axis(a.ax[1], n, lines_for(line));
  } else {
    stage_axis(a.ax[1], *V, ps.gv, n, inverse, kTileFloats / 16);
    const int line = a.ax[1].P * a.ax[1].W;
    free_axis(a.ax[0], m, lines_for(line));
  }
}

void set_signs(PassArgs& a, const Plan* U, const Plan* V) {
  if (U && U->signs) {
    a.ax[0].sign = U->signs;
    a.ax[0].sign_mod = U->d;
  }
  if (V && V->signs) {
    a.ax[1].sign = V->signs;
    a.ax[1].sign_mod = V->d;
  }
}

brq_status check_plan_device(const Plan* p) {
  if (!p) return BRQ_OK;
  int dev = -1;
  hipError_t e = rt_get_device(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "plan was created on device %d, current is %d",
                p->device, dev);
  return BRQ_OK;
}

brq_status check_quant(const brq_quant* q, int64_t n) {
  if (!q) return fail(BRQ_ERR_INVALID_ARGUMENT, "quantizer is NULL");
  if (q->kind != BRQ_ABSMAX && q->kind != BRQ_CODEBOOK_NORM)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "unknown quantizer kind %d", q->kind);
  if (q->bits < 2 || q->bits > 5) return fail(BRQ_ERR_INVALID_ARGUMENT, "bits must be 2..5");
  if (q->group <= 0 || n % q->group)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "group %d must divide n = %lld", q->group, (long long)n);
  if (((int64_t)q->group * q->bits) % 8)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "group*bits must be a multiple of 8");
  if (!is_pow2(q->group) || q->group < 64 || q->group > 1024)
    return fail(BRQ_ERR_UNSUPPORTED, "group must be a power of two in 64..1024");
  if (q->kind == BRQ_CODEBOOK_NORM) {
    const int L = 1 << q->bits;
    for (int i = 0; i < L; ++i)
      if (!std::isfinite(q->codebook[i]))
        return fail(BRQ_ERR_INVALID_ARGUMENT, "codebook entry %d is not finite", i);
    for (int i = 1; i < L; ++i)
      if (!(q->codebook[i] > q->codebook[i - 1]))
        return fail(BRQ_ERR_INVALID_ARGUMENT, "codebook must be strictly ascending");
  }
  return BRQ_OK;
}

void fill_quant(PassArgs& a, const brq_quant* q, int64_t n) {
  a.qkind = q->kind;
  a.bits = q->bits;
  a.group = q->group;
  a.nlev = 1 << q->bits;
  a.h = (float)((a.nlev - 1) * 0.5);
  a.sqrt_g = std::sqrt((float)q->group);
  for (int i = 0; i < kMaxLevels; ++i) {
    a.cent[i] = i < a.nlev && q->kind == BRQ_CODEBOOK_NORM ? q->codebook[i] : 0.f;
    a.tau[i] = 0.f;
  }
  if (q->kind == BRQ_CODEBOOK_NORM)
    for (int i = 0; i + 1 < a.nlev; ++i) a.tau[i] = (q->codebook[i] + q->codebook[i + 1]) * 0.5f;
  a.codes_ld = n * q->bits / 8;
  a.scales_ld = n / q->group;
}

// Run a forward transform (possibly none) from src into either dst or the
// quantizer.  ws holds the float32 intermediate when there is more than one pass.
brq_status run_forward(const Plan* U, const Plan* V, const void* src, int src_t, int64_t ld_src,
                       int64_t m, int64_t n, void* dst, int dst_t, int64_t ld_dst,
                       const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                       size_t ws_bytes, hipStream_t s) {
  std::vector<PassSpec> passes = plan_passes(U, V);
  // Can the quantizer ride on the last pass?  It needs contiguous whole groups
  // along the tile's columns: a right-side group ending at stride 1.
  bool fuse_q = false;
  if (q && !passes.empty()) {
    const PassSpec& last = passes.back();
    fuse_q = last.has_v && last.gv.S == 1 && (last.gv.P % q->group) == 0;
  }
  const size_t npass = passes.size() + ((q && !fuse_q) ? 1 : 0);
  const size_t need = npass > 1 ? (size_t)m * n * sizeof(float) : 0;
  if (need && (!ws || ws_bytes < need))
    return fail(BRQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);

  for (size_t i = 0; i < npass; ++i) {
    PassArgs a;
    std::memset(&a, 0, sizeof a);
    a.m = m;
    a.n = n;
    a.inverse = 0;
    if (i < passes.size()) {
      build_axes(a, passes[i], U, V, m, n, false);
    } else {  // stage-free quantizer pass
      free_axis(a.ax[0], m, 4);
      free_axis(a.ax[1], n, std::max(q->group, 256 - 256 % q->group));
      if (a.ax[1].P % q->group) a.ax[1].P = q->group;
    }
    if (i == 0) {
      set_signs(a, U, V);
      a.src = src;
      a.src_t = src_t;
      a.ld_src = ld_src;
    } else {
      a.src = ws;
      a.src_t = BRQ_F32;
      a.ld_src = n;
    }
    a.pro = PRO_LOAD;
    const bool last = (i + 1 == npass);
    if (last && q) {
      a.epi = EPI_QUANT;
      fill_quant(a, q, n);
      a.codes = codes;
      a.scales = scales;
    } else if (last) {
      a.epi = EPI_STORE;
      a.dst = dst;
      a.dst_t = dst_t;
      a.ld_dst = ld_dst;
    } else {
      a.epi = EPI_STORE;
      a.dst = ws;
      a.dst_t = BRQ_F32;
      a.ld_dst = n;
    }
    brq_status st = BRQ_OK;
    if (checked_launch(a, s, &st) != hipSuccess) return st;
  }
  return BRQ_OK;
}

// Inverse: optional dequant prologue in the first pass, inverse stages in
// reverse order, signs applied when storing the last pass.
brq_status run_inverse(const Plan* U, const Plan* V, const void* src, int src_t, int64_t ld_src,
                       const uint8_t* codes, const void* scales, const brq_quant* q, int64_t m,
                       int64_t n, void* dst, int dst_t, int64_t ld_dst, void* ws,
                       size_t ws_bytes, hipStream_t s) {
  std::vector<PassSpec> passes = plan_passes(U, V);
  std::reverse(passes.begin(), passes.end());
  const size_t npass = std::max<size_t>(passes.size(), 1);
  const size_t need = npass > 1 ? (size_t)m * n * sizeof(float) : 0;
  if (need && (!ws || ws_bytes < need))
    return fail(BRQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  for (size_t i = 0; i < npass; ++i) {
    PassArgs a;
    std::memset(&a, 0, sizeof a);
    a.m = m;
    a.n = n;
    a.inverse = 1;
    if (i < passes.size()) {
      build_axes(a, passes[i], U, V, m, n, true);
    } else {
      free_axis(a.ax[0], m, 4);
      free_axis(a.ax[1], n, 256);
    }
    if (i == 0) {
      if (q) {
        a.pro = PRO_DEQUANT;
        fill_quant(a, q, n);
        a.in_codes = codes;
        a.in_scales = scales;
      } else {
        a.pro = PRO_LOAD;
        a.src = src;
        a.src_t = src_t;
        a.ld_src = ld_src;
      }
    } else {
      a.pro = PRO_LOAD;
      a.src = ws;
      a.src_t = BRQ_F32;
      a.ld_src = n;
    }
    const bool last = (i + 1 == npass);
    a.epi = EPI_STORE;
    if (last) {
      set_signs(a, U, V);
      a.dst = dst;
      a.dst_t = dst_t;
      a.ld_dst = ld_dst;
    } else {
      a.dst = ws;
      a.dst_t = BRQ_F32;
      a.ld_dst = n;
    }
    brq_status st = BRQ_OK;
    if (checked_launch(a, s, &st) != hipSuccess) return st;
  }
  return BRQ_OK;
}

// Plans with dense blocks on either side run as stage passes into the
// float32 workspace (left side, then right side, in place), followed by a
// quantizer pass; the inverse is a dequantizer pass into the workspace and
// the inverse stages.
bool stage_sides_ok(const Plan* U, const Plan* V, int64_t m, int64_t n) {
  if (!U && !V) return false;
  if ((U && !sp_shape_ok(U, 1, m, n)) || (V && !sp_shape_ok(V, 0, m, n))) return false;
  return (U && U->mode != BRQ_HADAMARD) || (V && V->mode != BRQ_HADAMARD);
}

brq_status stage_fail(brq_status st, hipError_t he, size_t need, size_t have) {
  if (st == BRQ_ERR_HIP) return hip_fail(he, "stage pass launch");
  if (st == BRQ_ERR_WORKSPACE)
    return fail(st, "workspace of %zu bytes needed, %zu given", need, have);
  return st;
}

brq_status stage_rqp(const Plan* U, const Plan* V, const void* w, int wt, int64_t m, int64_t n,
                     int64_t ldw, const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  const size_t need = (size_t)m * n * sizeof(float);
  if (!ws || ws_bytes < need)
    return fail(BRQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  // Schedules ending in (16, 16) on both sides: stage passes for the earlier
  // stages, then pass B for the last four stages and the quantizer.
  const bool tail = fused_tail_supported(U, V, m, n, q) &&
                    reinterpret_cast<uintptr_t>(ws) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(codes) % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(scales) % 4 == 0;
  hipError_t he = hipSuccess;
  const void* src = w;
  int src_t = wt;
  int64_t ld = ldw;
  for (int side = 1; side >= 0; --side) {  // left, then right
    const Plan* p = side ? U : V;
    if (!p) continue;
    const brq_status st = sp_rotate_stages(p, side, 0, 0, tail ? p->nst - 2 : -1, src, src_t, ld,
                                           ws, BRQ_F32, n, m, n, ws, ws_bytes, s, &he);
    if (st != BRQ_OK) return stage_fail(st, he, need, ws_bytes);
    src = ws;
    src_t = BRQ_F32;
    ld = n;
  }
  if (tail) {
    const brq_status st = fused_tail_rqp(U, V, static_cast<const float*>(ws), m, n, q, codes,
                                         scales, s);
    if (st == BRQ_ERR_HIP) return hip_fail(hipGetLastError(), "pass B launch");
    if (st != BRQ_ERR_UNSUPPORTED) return st;
    return fail(BRQ_ERR_UNSUPPORTED, "pass B rejected a shape it reported as supported");
  }
  const brq_status st = rh_quant_only(ws, BRQ_F32, m, n, n, q, codes, scales, s);
  if (st == BRQ_ERR_HIP) return hip_fail(hipGetLastError(), "quantizer launch");
  if (st != BRQ_ERR_UNSUPPORTED) return st;
  return run_forward(nullptr, nullptr, ws, BRQ_F32, n, m, n, nullptr, 0, 0, q, codes, scales,
                     nullptr, 0, s);
}

brq_status stage_dequant(const Plan* U, const Plan* V, const uint8_t* codes, const void* scales,
                         const brq_quant* q, int64_t m, int64_t n, void* out, int ot, int64_t ldo,
                         void* ws, size_t ws_bytes, hipStream_t s) {
  const size_t need = (size_t)m * n * sizeof(float);
  if (!ws || ws_bytes < need)
    return fail(BRQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  brq_status st = run_inverse(nullptr, nullptr, nullptr, 0, 0, codes, scales, q, m, n, ws,
                              BRQ_F32, n, nullptr, 0, s);
  if (st != BRQ_OK) return st;
  hipError_t he = hipSuccess;
  for (int side = 0; side <= 1; ++side) {  // right, then left
    const Plan* p = side ? U : V;
    if (!p) continue;
    const bool last = side == 1 || !U;
    st = sp_rotate(p, side, 1, ws, BRQ_F32, n, last ? out : ws, last ? ot : BRQ_F32,
                   last ? ldo : n, m, n, ws, ws_bytes, s, &he);
    if (st != BRQ_OK) return stage_fail(st, he, need, ws_bytes);
  }
  return BRQ_OK;
}

brq_status rotate_common(const brq_plan* plan, int32_t side, int inverse, const void* x,
                         int32_t xt, int64_t ldx, void* y, int32_t yt, int64_t ldy, int64_t rows,
                         int64_t cols, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(BRQ_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (side != 0 && side != 1) return fail(BRQ_ERR_INVALID_ARGUMENT, "side must be 0 or 1");
  if (!valid_dtype(xt) || !valid_dtype(yt)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad dtype");
  if (rows < 0 || cols < 0) return fail(BRQ_ERR_INVALID_ARGUMENT, "negative shape");
  const Plan* p = &plan->p;
  if (side == 0 && (cols == 0 || cols % p->d))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "plan d = %d must divide cols = %lld", p->d,
                (long long)cols);
  if (side == 1 && rows != p->d)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "left side needs rows == d (%lld vs %d)",
                (long long)rows, p->d);
  if (ldx < cols || ldy < cols) return fail(BRQ_ERR_INVALID_ARGUMENT, "leading dimension < cols");
  if (rows == 0) return BRQ_OK;
  if (!x || !y) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if (x == y && (xt != yt || ldx != ldy))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "in place needs equal dtype and leading dimension");
  brq_status st = check_plan_device(p);
  if (st != BRQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Plan* U = side == 1 ? p : nullptr;
  const Plan* V = side == 0 ? p : nullptr;
  if (fast_paths() && rh_rotate_supported(p, side, xt, yt, rows, cols, ldx, ldy, x, y)) {
    st = rh_rotate(p, inverse, x, xt, ldx, y, yt, ldy, rows, cols, s);
    return st == BRQ_OK ? st : hip_fail(hipGetLastError(), "row Hadamard launch");
  }
  if (fast_paths() && !inverse && fused_rotate_supported(U, V, xt, yt, rows, cols, ldx, ldy, x, y))
    return fused_rotate(U, V, x, xt, ldx, y, yt, ldy, rows, cols, s) == hipSuccess
               ? BRQ_OK
               : hip_fail(hipGetLastError(), "fused rotate launch");
  if (fast_paths() && sp_rotate_supported(p, side, rows, cols)) {
    hipError_t he = hipSuccess;
    st = sp_rotate(p, side, inverse, x, xt, ldx, y, yt, ldy, rows, cols, ws, ws_bytes, s, &he);
    if (st != BRQ_ERR_UNSUPPORTED)
      return stage_fail(st, he, (size_t)rows * cols * sizeof(float), ws_bytes);
  }
  if (!inverse)
    return run_forward(U, V, x, xt, ldx, rows, cols, y, yt, ldy, nullptr, nullptr, nullptr, ws,
                       ws_bytes, s);
  return run_inverse(U, V, x, xt, ldx, nullptr, nullptr, nullptr, rows, cols, y, yt, ldy, ws,
                     ws_bytes, s);
}

// ---------------------------------------------------------------- Lloyd-Max

double npdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }
double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }

// Residual of the centroid condition on the positive half (even level count).
void lm_residual(const std::vector<double>& c, std::vector<double>& r) {
  const size_t h = c.size();
  r.resize(h);
  for (size_t k = 0; k < h; ++k) {
    const double a = k == 0 ? 0.0 : 0.5 * (c[k - 1] + c[k]);
    const double b = k + 1 == h ? INFINITY : 0.5 * (c[k] + c[k + 1]);
    const double pa = npdf(a), pb = std::isinf(b) ? 0.0 : npdf(b);
    const double mass = upper_tail(a) - (std::isinf(b) ? 0.0 : upper_tail(b));
    r[k] = c[k] - (pa - pb) / mass;
  }
}

}  // namespace
}  // namespace brq

using namespace brq;

extern "C" {

const char* brq_status_string(brq_status s) {
  switch (s) {
    case BRQ_OK: return "BRQ_OK";
    case BRQ_ERR_INVALID_ARGUMENT: return "BRQ_ERR_INVALID_ARGUMENT";
    case BRQ_ERR_UNSUPPORTED: return "BRQ_ERR_UNSUPPORTED";
    case BRQ_ERR_ALIGNMENT: return "BRQ_ERR_ALIGNMENT";
    case BRQ_ERR_WORKSPACE: return "BRQ_ERR_WORKSPACE";
    case BRQ_ERR_HIP: return "BRQ_ERR_HIP";
  }
  return "BRQ_UNKNOWN_STATUS";
}

const char* brq_last_error(void) { return g_last_error.c_str(); }

int32_t brq_version(void) { return 100; }

brq_status brq_set_path(int32_t path) {
  g_last_error.clear();
  if (path != BRQ_PATH_AUTO && path != BRQ_PATH_TILE)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "unknown path %d", path);
  g_path.store(path, std::memory_order_relaxed);
  return BRQ_OK;
}

brq_status brq_plan_create(brq_plan** out, int32_t d, int32_t n_stages, const int32_t* radix,
                           const float* blocks, int32_t mode, const int8_t* signs) {
  g_last_error.clear();
  if (!out) return fail(BRQ_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (d < 2) return fail(BRQ_ERR_INVALID_ARGUMENT, "d must be >= 2");
  if (n_stages < 1 || n_stages > kMaxStages)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "n_stages must be 1..%d", kMaxStages);
  if (!radix) return fail(BRQ_ERR_INVALID_ARGUMENT, "radix is NULL");
  if (mode != BRQ_HADAMARD && mode != BRQ_SHARED && mode != BRQ_PER_GROUP)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "unknown block mode %d", mode);
  int64_t prod = 1;
  for (int t = 0; t < n_stages; ++t) {
    if (radix[t] < 2) return fail(BRQ_ERR_INVALID_ARGUMENT, "radix[%d] = %d < 2", t, radix[t]);
    prod *= radix[t];
    if (prod > (int64_t)1 << 40) break;
  }
  if (prod != d)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "product of radices (%lld) != d (%d)", (long long)prod,
                d);
  if (d > (1 << 22)) return fail(BRQ_ERR_UNSUPPORTED, "d > 2^22");
  for (int t = 0; t < n_stages; ++t) {
    if (radix[t] > 64) return fail(BRQ_ERR_UNSUPPORTED, "radix[%d] = %d > 64", t, radix[t]);
    if (mode == BRQ_HADAMARD && !is_pow2(radix[t]))
      return fail(BRQ_ERR_UNSUPPORTED, "Hadamard radix %d is not a power of two", radix[t]);
  }
  if (mode != BRQ_HADAMARD && !blocks)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "blocks are required for this mode");
  if (signs)
    for (int i = 0; i < d; ++i)
      if (signs[i] != 1 && signs[i] != -1)
        return fail(BRQ_ERR_INVALID_ARGUMENT, "signs[%d] = %d is not +-1", i, (int)signs[i]);

  brq_plan* h = new (std::nothrow) brq_plan;
  if (!h) return fail(BRQ_ERR_HIP, "host allocation failed");
  Plan& p = h->p;
  p.d = d;
  p.nst = n_stages;
  p.mode = mode;
  size_t total = 0;
  for (int t = 0; t < n_stages; ++t) p.radix[t] = radix[t];
  for (int t = 0; t < n_stages; ++t) {
    int64_t s = 1;
    for (int u = t + 1; u < n_stages; ++u) s *= radix[u];
    p.stride[t] = (int)s;
    p.blk_off[t] = total;
    const size_t bb = (size_t)radix[t] * radix[t];
    if (mode == BRQ_SHARED) total += bb;
    else if (mode == BRQ_PER_GROUP) total += (size_t)(d / radix[t]) * bb;
  }
  hipError_t e = rt_get_device(&p.device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  std::vector<float> host_t;
  if (total) {
    e = rt_malloc((void**)&p.blk, total * sizeof(float));
    if (e == hipSuccess) e = rt_malloc((void**)&p.blkT, total * sizeof(float));
    if (e == hipSuccess) e = rt_copy_to_device(p.blk, blocks, total * sizeof(float));
    if (e == hipSuccess) {
      host_t.resize(total);
      for (int t = 0; t < n_stages; ++t) {
        const int b = radix[t];
        const size_t nb = mode == BRQ_SHARED ? 1 : (size_t)(d / b);
        for (size_t g = 0; g < nb; ++g) {
          const float* src = blocks + p.blk_off[t] + g * b * b;
          float* dst = host_t.data() + p.blk_off[t] + g * b * b;
          for (int j = 0; j < b; ++j)
            for (int k = 0; k < b; ++k) dst[k * b + j] = src[j * b + k];
        }
      }
      e = rt_copy_to_device(p.blkT, host_t.data(), total * sizeof(float));
    }
  }
  if (e == hipSuccess && signs) {
    std::vector<float> sf(d);
    for (int i = 0; i < d; ++i) sf[i] = (float)signs[i];
    e = rt_malloc((void**)&p.signs, d * sizeof(float));
    if (e == hipSuccess) e = rt_copy_to_device(p.signs, sf.data(), d * sizeof(float));
    if (e == hipSuccess && mode == BRQ_HADAMARD) {
      const float sc = 1.0f / std::sqrt((float)d);
      for (int i = 0; i < d; ++i) sf[i] *= sc;
      e = rt_malloc((void**)&p.signs_s, d * sizeof(float));
      if (e == hipSuccess) e = rt_copy_to_device(p.signs_s, sf.data(), d * sizeof(float));
    }
  }
  if (signs) h->signs.assign(signs, signs + d);
  if (e == hipSuccess) e = fused_prepare(p, blocks, signs);
  if (e != hipSuccess) {
    brq_status st = hip_fail(e, "plan device setup");
    brq_plan_destroy(h);
    return st;
  }
  *out = h;
  return BRQ_OK;
}

namespace {
brq_status harp_job_check(int32_t b, int64_t ngroups, const int8_t* theta_q, float scale, const float* base,
                          const float* blocks) {
  if (b < 2 || b > 64) return fail(BRQ_ERR_INVALID_ARGUMENT, "radix %d is not in 2..64", b);
  if (ngroups < 0 || ngroups >= ((int64_t)1 << 31))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "ngroups %lld is not in 0..2^31-1", (long long)ngroups);
  if (!base && !is_pow2(b))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "radix %d needs a base mixer (not a power of two)", b);
  if (!std::isfinite(scale)) return fail(BRQ_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (ngroups > 0 && (!theta_q || !blocks)) return fail(BRQ_ERR_INVALID_ARGUMENT, "theta_q or blocks is NULL");
  return BRQ_OK;
}
}  // namespace

brq_status brq_harp_blocks_batch(int32_t n_jobs, const brq_harp_job* jobs, void* stream) {
  g_last_error.clear();
  if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad job list");
  for (int i = 0; i < n_jobs; ++i) {
    const brq_harp_job& j = jobs[i];
    const brq_status st = harp_job_check(j.b, j.ngroups, j.theta_q, j.scale, j.base, j.blocks);
    if (st != BRQ_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // batchable jobs, largest radix first (their long eliminations start first)
  std::vector<int> order;
  for (int i = 0; i < n_jobs; ++i)
    if (jobs[i].ngroups > 0) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return jobs[x].b > jobs[y].b; });
  HarpBatch bt;
  std::memset(&bt, 0, sizeof bt);
  auto flush = [&]() -> brq_status {
    if (bt.n == 0) return BRQ_OK;
    const int tok = prof_begin("harp blocks batch", s);
    const hipError_t e = launch_harp_batch(bt, s);
    prof_end(tok, s);
    std::memset(&bt, 0, sizeof bt);
    return e == hipSuccess ? BRQ_OK : hip_fail(e, "HARP batch launch");
  };
  for (int i : order) {
    const brq_harp_job& j = jobs[i];
    if (!harp_batchable(j.b)) {
      const brq_status st = brq_harp_blocks(j.b, j.ngroups, j.theta_q, j.scale, j.base, j.blocks, stream);
      if (st != BRQ_OK) return st;
      continue;
    }
    if (bt.n == kHpMaxJobs || bt.first[bt.n] + j.ngroups >= ((int64_t)1 << 31)) {
      const brq_status st = flush();
      if (st != BRQ_OK) return st;
    }
    HarpArgs& a = bt.job[bt.n];
    a.b = j.b;
    a.np = harp_params(j.b);
    a.ngroups = j.ngroups;
    a.theta = j.theta_q;
    a.scale = j.scale;
    a.base = j.base;
    a.out = j.blocks;
    bt.first[bt.n + 1] = bt.first[bt.n] + j.ngroups;
    ++bt.n;
  }
  return flush();
}

brq_status brq_harp_blocks(int32_t b, int64_t ngroups, const int8_t* theta_q, float scale,
                           const float* base, float* blocks, void* stream) {
  g_last_error.clear();
  if (b < 2 || b > 64) return fail(BRQ_ERR_INVALID_ARGUMENT, "radix %d is not in 2..64", b);
  if (ngroups < 0 || ngroups >= ((int64_t)1 << 31))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "ngroups %lld is not in 0..2^31-1", (long long)ngroups);
  if (!base && !is_pow2(b))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "radix %d needs a base mixer (not a power of two)", b);
  if (!std::isfinite(scale)) return fail(BRQ_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (ngroups == 0) return BRQ_OK;
  if (!theta_q || !blocks) return fail(BRQ_ERR_INVALID_ARGUMENT, "theta_q or blocks is NULL");
  HarpArgs a;
  a.b = b;
  a.np = harp_params(b);
  a.ngroups = ngroups;
  a.theta = theta_q;
  a.scale = scale;
  a.base = base;
  a.out = blocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char name[48];
  snprintf(name, sizeof name, "harp blocks %s b%d", b == 2 ? "Givens" : "Cayley", b);
  const int tok = prof_begin(name, s);
  const hipError_t e = launch_harp(a, s);
  prof_end(tok, s);
  return e == hipSuccess ? BRQ_OK : hip_fail(e, "HARP block launch");
}

brq_status brq_plan_create_harp(brq_plan** out, int32_t d, int32_t n_stages, const int32_t* radix,
                                const int8_t* theta_q, const float* scales, const float* bases,
                                const int8_t* signs) {
  g_last_error.clear();
  if (!out) return fail(BRQ_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (n_stages < 1 || n_stages > kMaxStages)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "n_stages must be 1..%d", kMaxStages);
  if (!radix || !theta_q || !scales)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "radix, theta_q or scales is NULL");
  int64_t prod = 1, nparams = 0, nblk = 0, nbase = 0;
  for (int t = 0; t < n_stages; ++t) {
    if (radix[t] < 2 || radix[t] > 64)
      return fail(BRQ_ERR_INVALID_ARGUMENT, "radix[%d] = %d is not in 2..64", t, radix[t]);
    if (!bases && !is_pow2(radix[t]))
      return fail(BRQ_ERR_INVALID_ARGUMENT, "radix[%d] = %d needs a base mixer", t, radix[t]);
    prod *= radix[t];
    if (prod > (int64_t)1 << 22) return fail(BRQ_ERR_UNSUPPORTED, "d > 2^22");
  }
  if (prod != d) return fail(BRQ_ERR_INVALID_ARGUMENT, "product of radices != d (%d)", d);
  for (int t = 0; t < n_stages; ++t) {
    const int64_t ng = d / radix[t];
    nparams += ng * harp_params(radix[t]);
    nblk += ng * radix[t] * radix[t];
    nbase += (int64_t)radix[t] * radix[t];
  }
  // device copies of the parameters (and bases), the blocks built there, then
  // back to the host for the ordinary plan set-up
  int8_t* dth = nullptr;
  float* dbase = nullptr;
  float* dblk = nullptr;
  std::vector<float> hblk((size_t)nblk);
  hipError_t e = rt_malloc((void**)&dth, (size_t)nparams);
  if (e == hipSuccess) e = rt_malloc((void**)&dblk, (size_t)nblk * sizeof(float));
  if (e == hipSuccess && bases) e = rt_malloc((void**)&dbase, (size_t)nbase * sizeof(float));
  if (e == hipSuccess) e = rt_copy_to_device(dth, theta_q, (size_t)nparams);
  if (e == hipSuccess && bases) e = rt_copy_to_device(dbase, bases, (size_t)nbase * sizeof(float));
  brq_status st = BRQ_OK;
  if (e == hipSuccess) {  // every stage in one batch
    std::vector<brq_harp_job> jobs((size_t)n_stages);
    int64_t poff = 0, boff = 0, goff = 0;
    for (int t = 0; t < n_stages; ++t) {
      const int b = radix[t];
      const int64_t ng = d / b;
      jobs[t] = brq_harp_job{b, ng, dth + poff, scales[t], bases ? dbase + goff : nullptr, dblk + boff};
      poff += ng * harp_params(b);
      boff += ng * b * b;
      goff += (int64_t)b * b;
    }
    st = brq_harp_blocks_batch(n_stages, jobs.data(), nullptr);
  }
  if (e == hipSuccess && st == BRQ_OK) e = rt_copy_to_host(hblk.data(), dblk, (size_t)nblk * sizeof(float));
  rt_free(dth);
  rt_free(dbase);
  rt_free(dblk);
  if (st != BRQ_OK) return st;
  if (e != hipSuccess) return hip_fail(e, "HARP plan set-up");
  st = brq_plan_create(out, d, n_stages, radix, hblk.data(), BRQ_PER_GROUP, signs);
  if (st == BRQ_OK) {
    brq_plan* h = *out;
    h->harp = true;
    h->theta.assign(theta_q, theta_q + nparams);
    h->scales.assign(scales, scales + n_stages);
    if (bases) h->bases.assign(bases, bases + nbase);
  }
  return st;
}

// ---- plan serialisation ------------------------------------------------------
//
// Little-endian byte image: "BRQP", u32 version 1, u32 kind (0: blocks,
// 1: HARP parameters), i32 d, i32 n_stages, i32 mode, u32 flags (bit 0 signs,
// bit 1 base mixers), i32 radix[n_stages]; kind 0: float32 blocks in
// brq_plan_create's layout; kind 1: float32 scales[n_stages], float32 base
// mixers (flag 1), int8 parameters; int8 signs (flag 0); u64 FNV-1a hash of
// every byte before it.

}  // extern "C"

namespace brq {
namespace {

constexpr uint32_t kSerVersion = 1;

struct ByteWriter {
  uint8_t* buf;
  size_t cap, n = 0;
  void put(const void* p, size_t k) {
    if (buf && n + k <= cap) std::memcpy(buf + n, p, k);
    n += k;
  }
  template <typename T> void val(T v) { put(&v, sizeof v); }
};

uint64_t fnv1a(const uint8_t* p, size_t n) {
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

size_t plan_block_floats(const Plan& p) {
  size_t total = 0;
  for (int t = 0; t < p.nst; ++t) {
    const size_t bb = (size_t)p.radix[t] * p.radix[t];
    if (p.mode == BRQ_SHARED) total += bb;
    else if (p.mode == BRQ_PER_GROUP) total += (size_t)(p.d / p.radix[t]) * bb;
  }
  return total;
}

}  // namespace
}  // namespace brq

extern "C" {

brq_status brq_plan_serialize(const brq_plan* plan, void* buf, size_t cap, size_t* size) {
  g_last_error.clear();
  if (!plan || !size) return fail(BRQ_ERR_INVALID_ARGUMENT, "plan or size is NULL");
  const Plan& p = plan->p;
  std::vector<float> blocks;
  if (!plan->harp && p.blk) {  // fetch the blocks only when writing
    if (buf) {
      blocks.resize(plan_block_floats(p));
      const hipError_t e = rt_copy_to_host(blocks.data(), p.blk, blocks.size() * sizeof(float));
      if (e != hipSuccess) return hip_fail(e, "plan block copy");
    }
  }
  const uint32_t flags = (plan->signs.empty() ? 0u : 1u) | (plan->bases.empty() ? 0u : 2u);
  ByteWriter w{static_cast<uint8_t*>(buf), cap};
  w.put("BRQP", 4);
  w.val<uint32_t>(kSerVersion);
  w.val<uint32_t>(plan->harp ? 1u : 0u);
  w.val<int32_t>(p.d);
  w.val<int32_t>(p.nst);
  w.val<int32_t>(p.mode);
  w.val<uint32_t>(flags);
  w.put(p.radix, sizeof(int32_t) * p.nst);
  if (plan->harp) {
    w.put(plan->scales.data(), sizeof(float) * plan->scales.size());
    w.put(plan->bases.data(), sizeof(float) * plan->bases.size());
    w.put(plan->theta.data(), plan->theta.size());
  } else if (buf) {
    w.put(blocks.data(), sizeof(float) * blocks.size());
  } else {
    w.n += sizeof(float) * plan_block_floats(p);
  }
  w.put(plan->signs.data(), plan->signs.size());
  const size_t body = w.n;
  w.n += sizeof(uint64_t);
  *size = w.n;
  if (!buf) return BRQ_OK;
  if (cap < w.n) return fail(BRQ_ERR_INVALID_ARGUMENT, "buffer of %zu bytes < %zu", cap, w.n);
  const uint64_t h = fnv1a(static_cast<uint8_t*>(buf), body);
  std::memcpy(static_cast<uint8_t*>(buf) + body, &h, sizeof h);
  return BRQ_OK;
}

brq_status brq_plan_deserialize(brq_plan** out, const void* buf, size_t size) {
  g_last_error.clear();
  if (!out || !buf) return fail(BRQ_ERR_INVALID_ARGUMENT, "out or buf is NULL");
  *out = nullptr;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  size_t at = 0;
  auto take = [&](void* dst, size_t k) {
    if (at + k > size) return false;
    std::memcpy(dst, b + at, k);
    at += k;
    return true;
  };
  char magic[4];
  uint32_t version = 0, kind = 0, flags = 0;
  int32_t d = 0, nst = 0, mode = 0;
  if (size < 8 + sizeof(uint64_t)) return fail(BRQ_ERR_INVALID_ARGUMENT, "image too short");
  uint64_t h_stored;
  std::memcpy(&h_stored, b + size - sizeof h_stored, sizeof h_stored);
  if (fnv1a(b, size - sizeof h_stored) != h_stored)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "image hash mismatch (corrupt or truncated)");
  size -= sizeof h_stored;
  if (!take(magic, 4) || std::memcmp(magic, "BRQP", 4))
    return fail(BRQ_ERR_INVALID_ARGUMENT, "not a plan image");
  if (!take(&version, 4) || version != kSerVersion)
    return fail(BRQ_ERR_UNSUPPORTED, "plan image version %u", version);
  if (!take(&kind, 4) || !take(&d, 4) || !take(&nst, 4) || !take(&mode, 4) || !take(&flags, 4) ||
      kind > 1 || nst < 1 || nst > kMaxStages)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "malformed plan header");
  int32_t radix[kMaxStages];
  if (!take(radix, sizeof(int32_t) * nst)) return fail(BRQ_ERR_INVALID_ARGUMENT, "truncated radices");
  int64_t prod = 1, nparams = 0, nbase = 0, nblk = 0;
  for (int t = 0; t < nst; ++t) {
    if (radix[t] < 2 || radix[t] > 64) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad radix %d", radix[t]);
    prod *= radix[t];
    if (prod > ((int64_t)1 << 22)) return fail(BRQ_ERR_INVALID_ARGUMENT, "d too large");
  }
  if (prod != d) return fail(BRQ_ERR_INVALID_ARGUMENT, "radices do not multiply to d");
  for (int t = 0; t < nst; ++t) {
    const int64_t bb = (int64_t)radix[t] * radix[t];
    nparams += (d / radix[t]) * harp_params(radix[t]);
    nbase += bb;
    nblk += mode == BRQ_SHARED ? bb : mode == BRQ_PER_GROUP ? (d / radix[t]) * bb : 0;
  }
  std::vector<float> scales, bases, blocks;
  std::vector<int8_t> theta, signs;
  if (kind == 1) {
    scales.resize(nst);
    if (!take(scales.data(), sizeof(float) * nst)) return fail(BRQ_ERR_INVALID_ARGUMENT, "truncated scales");
    if (flags & 2u) {
      bases.resize(nbase);
      if (!take(bases.data(), sizeof(float) * nbase)) return fail(BRQ_ERR_INVALID_ARGUMENT, "truncated bases");
    }
    theta.resize(nparams);
    if (!take(theta.data(), nparams)) return fail(BRQ_ERR_INVALID_ARGUMENT, "truncated parameters");
  } else if (nblk) {
    blocks.resize(nblk);
    if (!take(blocks.data(), sizeof(float) * nblk)) return fail(BRQ_ERR_INVALID_ARGUMENT, "truncated blocks");
  }
  if (flags & 1u) {
    signs.resize(d);
    if (!take(signs.data(), d)) return fail(BRQ_ERR_INVALID_ARGUMENT, "truncated signs");
  }
  if (at != size) return fail(BRQ_ERR_INVALID_ARGUMENT, "%zu trailing bytes", size - at);
  const int8_t* sg = signs.empty() ? nullptr : signs.data();
  if (kind == 1)
    return brq_plan_create_harp(out, d, nst, radix, theta.data(), scales.data(),
                                bases.empty() ? nullptr : bases.data(), sg);
  return brq_plan_create(out, d, nst, radix, blocks.empty() ? nullptr : blocks.data(), mode, sg);
}

brq_status brq_plan_destroy(brq_plan* plan) {
  if (!plan) return BRQ_OK;
  Plan& p = plan->p;
  rt_free(p.blk);
  rt_free(p.blkT);
  rt_free(p.signs);
  rt_free(p.signs_s);
  fused_release(p);
  delete plan;
  return BRQ_OK;
}

int32_t brq_plan_dim(const brq_plan* plan) { return plan ? plan->p.d : 0; }

size_t brq_workspace_bytes(const brq_plan* left, const brq_plan* right, int64_t m, int64_t n) {
  if (m <= 0 || n <= 0) return 0;
  if (!left && !right) return (size_t)m * n * sizeof(float);  // stand-alone quantizer pass
  return (size_t)m * n * sizeof(float);
}

brq_status brq_rotate(const brq_plan* plan, int32_t side, const void* x, int32_t xt, int64_t ldx,
                      void* y, int32_t yt, int64_t ldy, int64_t rows, int64_t cols, void* ws,
                      size_t ws_bytes, void* stream) {
  return rotate_common(plan, side, 0, x, xt, ldx, y, yt, ldy, rows, cols, ws, ws_bytes, stream);
}

brq_status brq_rotate_inverse(const brq_plan* plan, int32_t side, const void* x, int32_t xt,
                              int64_t ldx, void* y, int32_t yt, int64_t ldy, int64_t rows,
                              int64_t cols, void* ws, size_t ws_bytes, void* stream) {
  return rotate_common(plan, side, 1, x, xt, ldx, y, yt, ldy, rows, cols, ws, ws_bytes, stream);
}

brq_status brq_rotate_quantize_pack(const brq_plan* left, const brq_plan* right, const void* w,
                                    int32_t wt, int64_t m, int64_t n, int64_t ldw,
                                    const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                                    size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!valid_dtype(wt)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad dtype");
  if (m < 0 || n <= 0) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad shape");
  if (ldw < n) return fail(BRQ_ERR_INVALID_ARGUMENT, "leading dimension < n");
  brq_status st = check_quant(q, n);
  if (st != BRQ_OK) return st;
  const Plan* U = left ? &left->p : nullptr;
  const Plan* V = right ? &right->p : nullptr;
  if (U && U->d != m)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "left plan d = %d != m = %lld", U->d, (long long)m);
  if (V && n % V->d)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "right plan d = %d does not divide n", V->d);
  if (m == 0) return BRQ_OK;
  if (!w || !codes || !scales) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if ((st = check_plan_device(U)) != BRQ_OK) return st;
  if ((st = check_plan_device(V)) != BRQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fast_paths() && fused_rqp_supported(U, V, wt, m, n, ldw, w, q)) {
    st = fused_rqp(U, V, w, wt, m, n, ldw, q, codes, scales, ws, ws_bytes, s);
    if (st != BRQ_ERR_UNSUPPORTED) return st;
  }
  if (fast_paths() && rh_quant_supported(U, V, wt, m, n, ldw, w, q)) {
    st = rh_rqp(V, w, wt, m, n, ldw, q, codes, scales, s);
    if (st == BRQ_ERR_HIP) return hip_fail(hipGetLastError(), "row Hadamard launch");
    if (st != BRQ_ERR_UNSUPPORTED) return st;
  }
  if (fast_paths() && !U && !V) {
    st = rh_quant_only(w, wt, m, n, ldw, q, codes, scales, s);
    if (st == BRQ_ERR_HIP) return hip_fail(hipGetLastError(), "quantizer launch");
    if (st != BRQ_ERR_UNSUPPORTED) return st;
  }
  if (fast_paths() && stage_sides_ok(U, V, m, n))
    return stage_rqp(U, V, w, wt, m, n, ldw, q, codes, scales, ws, ws_bytes, s);
  return run_forward(U, V, w, wt, ldw, m, n, nullptr, 0, 0, q, codes, scales, ws, ws_bytes, s);
}

brq_status brq_dequant_unrotate(const brq_plan* left, const brq_plan* right, const uint8_t* codes,
                                const void* scales, const brq_quant* q, int64_t m, int64_t n,
                                void* out, int32_t ot, int64_t ldo, void* ws, size_t ws_bytes,
                                void* stream) {
  g_last_error.clear();
  if (!valid_dtype(ot)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad dtype");
  if (m < 0 || n <= 0) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad shape");
  if (ldo < n) return fail(BRQ_ERR_INVALID_ARGUMENT, "leading dimension < n");
  brq_status st = check_quant(q, n);
  if (st != BRQ_OK) return st;
  const Plan* U = left ? &left->p : nullptr;
  const Plan* V = right ? &right->p : nullptr;
  if (U && U->d != m)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "left plan d = %d != m = %lld", U->d, (long long)m);
  if (V && n % V->d)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "right plan d = %d does not divide n", V->d);
  if (m == 0) return BRQ_OK;
  if (!codes || !scales || !out) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if ((st = check_plan_device(U)) != BRQ_OK) return st;
  if ((st = check_plan_device(V)) != BRQ_OK) return st;
  if (fast_paths() && !U && rh_plan_ok(V) && q->group <= 1024) {
    st = rh_dequant(V, codes, scales, q, m, n, out, ot, ldo, static_cast<hipStream_t>(stream));
    if (st == BRQ_ERR_HIP) return hip_fail(hipGetLastError(), "row Hadamard launch");
    if (st != BRQ_ERR_UNSUPPORTED) return st;
  }
  if (fast_paths() && stage_sides_ok(U, V, m, n))
    return stage_dequant(U, V, codes, scales, q, m, n, out, ot, ldo, ws, ws_bytes,
                         static_cast<hipStream_t>(stream));
  return run_inverse(U, V, nullptr, 0, 0, codes, scales, q, m, n, out, ot, ldo, ws, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

// The fused re-quantizer takes the call (no workspace needed).
static bool requant_fused(const brq_plan* right, const brq_quant* q_in, const brq_quant* q_out,
                          int64_t m, int64_t n) {
  const Plan* V = right ? &right->p : nullptr;
  return fast_paths() && V && rh_plan_ok(V) && V->d >= 64 && V->d <= 256 && n % V->d == 0 &&
         q_out->kind == BRQ_ABSMAX && q_out->group <= 1024 && q_in->group <= 1024 &&
         m * (n / V->d) <= kRhMaxChunks;
}

size_t brq_requant_workspace_bytes(const brq_plan* right, const brq_quant* q_in,
                                   const brq_quant* q_out, int64_t m, int64_t n) {
  if (m <= 0 || n <= 0 || !q_in || !q_out) return 0;
  if (requant_fused(right, q_in, q_out, m, n)) return 0;
  return 2 * (size_t)m * n * sizeof(float);
}

brq_status brq_requant(const brq_plan* right, const uint8_t* codes, const void* scales,
                       const brq_quant* q_in, int64_t m, int64_t n, const brq_quant* q_out,
                       uint8_t* codes_out, void* scales_out, void* ws, size_t ws_bytes,
                       void* stream) {
  g_last_error.clear();
  if (m < 0 || n <= 0) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad shape");
  brq_status st = check_quant(q_in, n);
  if (st != BRQ_OK) return st;
  if ((st = check_quant(q_out, n)) != BRQ_OK) return st;
  if (q_out->kind != BRQ_ABSMAX)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "the downstream quantizer is absmax");
  const Plan* V = right ? &right->p : nullptr;
  if (V && n % V->d)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "right plan d = %d does not divide n", V->d);
  if (m == 0) return BRQ_OK;
  if (!codes || !scales || !codes_out || !scales_out)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if ((st = check_plan_device(V)) != BRQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (requant_fused(right, q_in, q_out, m, n)) {
    st = rh_requant(V, codes, scales, q_in, m, n, q_out, codes_out, scales_out, s);
    if (st == BRQ_ERR_HIP) return hip_fail(hipGetLastError(), "re-quantizer launch");
    if (st != BRQ_ERR_UNSUPPORTED) return st;
  }
  // composed: restore into the workspace, then the quantizer on its own
  const size_t half = (size_t)m * n * sizeof(float);
  if (!ws || ws_bytes < 2 * half)
    return fail(BRQ_ERR_WORKSPACE, "workspace of %zu bytes < %zu", ws_bytes, 2 * half);
  float* restored = static_cast<float*>(ws);
  void* inner = static_cast<char*>(ws) + half;
  st = brq_dequant_unrotate(nullptr, right, codes, scales, q_in, m, n, restored, BRQ_F32, n, inner,
                            half, stream);
  if (st != BRQ_OK) return st;
  return brq_rotate_quantize_pack(nullptr, nullptr, restored, BRQ_F32, m, n, n, q_out, codes_out,
                                  scales_out, inner, half, stream);
}

// ---- quantized linear layer at decode ----------------------------------------

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Split the input index so that a few tokens still fill the GPU: about 2048
// workgroups (measured on the 70B down projection: more, shorter workgroups
// beat fewer with longer load pipelines).  The split count does not depend
// on the pointers, so the workspace size is known before the call.
int ql_splits(int64_t T, int64_t m, int64_t n, int bits, int group) {
  const int kind = ql_kind(T, m, n, bits, group, true);
  if (kind == kQlGemm) return ql_gemm_splits(T, n);
  const int tm = ql_kind_tm(kind, T, bits, group);
  const int64_t tt = kQlTok * tm;
  const int64_t base = (m / (kQlOut * ql_kind_tn(kind, tm))) * ((T + tt - 1) / tt);
  int64_t s = (2048 + base - 1) / base;
  const int64_t ng = n / group;
  if (s > ng) s = ng;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

struct QlLayout {
  size_t xt_off, part_off, z_off, rot_off, total, rot_bytes;
  int splits;
  int64_t kc;
};

QlLayout ql_layout(const Plan* U, const Plan* V, const brq_quant* q, int64_t T, int64_t m,
                   int64_t n) {
  QlLayout L;
  L.splits = ql_splits(T, m, n, q->bits, q->group);
  // the staged kernels' splits hold whole chunks
  const int unit = ql_kind(T, m, n, q->bits, q->group, true) == kQlGemm ? kQlGemmChunk
                   : n % kQlChunk == 0                                  ? kQlChunk
                                                                        : q->group;
  const int64_t nu = n / unit;
  if (L.splits > nu) L.splits = (int)nu;
  L.kc = ((nu + L.splits - 1) / L.splits) * unit;
  L.splits = (int)((n + L.kc - 1) / L.kc);
  size_t at = 0;
  L.xt_off = at;
  if (V) at += align256((size_t)T * n * 2);
  L.part_off = at;
  at += align256((size_t)L.splits * T * m * sizeof(float));
  L.z_off = at;
  if (U) at += align256((size_t)T * m * sizeof(float));
  L.rot_off = at;
  // the rotations' own float32 intermediate (X~ written in a 16-bit type,
  // Y in the caller's type)
  const size_t rin = V ? (size_t)T * n * sizeof(float) : 0;
  const size_t rout = U ? (size_t)T * m * sizeof(float) : 0;
  L.rot_bytes = rin > rout ? rin : rout;
  L.total = at + L.rot_bytes;
  return L;
}

}  // namespace

size_t brq_qlinear_workspace_bytes(const brq_plan* left, const brq_plan* right,
                                   const brq_quant* q, int64_t T, int64_t m, int64_t n) {
  if (!q || T <= 0 || m <= 0 || n <= 0 || q->group <= 0 || n % q->group) return 0;
  return ql_layout(left ? &left->p : nullptr, right ? &right->p : nullptr, q, T, m, n).total;
}

brq_status brq_qlinear(const brq_plan* left, const brq_plan* right, const void* x, int32_t xt,
                       int64_t ldx, int64_t T, const uint8_t* codes, const void* scales,
                       const brq_quant* q, int64_t m, int64_t n, void* y, int32_t yt, int64_t ldy,
                       void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (xt != BRQ_F16 && xt != BRQ_BF16)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "activations must be f16 or bf16");
  if (!valid_dtype(yt)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad output dtype");
  if (T < 0 || m <= 0 || n <= 0 || ldx < n || ldy < m)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "bad shape or leading dimension");
  brq_status st = check_quant(q, n);
  if (st != BRQ_OK) return st;
  if (q->kind != BRQ_ABSMAX) return fail(BRQ_ERR_INVALID_ARGUMENT, "the weight must be absmax-quantized");
  if (q->group != 64 && q->group != 128) return fail(BRQ_ERR_UNSUPPORTED, "weight groups of 64 or 128");
  const Plan* U = left ? &left->p : nullptr;
  const Plan* V = right ? &right->p : nullptr;
  if (U && U->d != m) return fail(BRQ_ERR_INVALID_ARGUMENT, "left plan d = %d != m", U->d);
  if (V && n % V->d) return fail(BRQ_ERR_INVALID_ARGUMENT, "right plan d = %d does not divide n", V->d);
  if (m % (kQlOut * ql_tn(ql_tm(T))))
    return fail(BRQ_ERR_UNSUPPORTED, "m must be a multiple of %d", kQlOut * ql_tn(ql_tm(T)));
  if (T == 0) return BRQ_OK;
  if (!x || !codes || !scales || !y) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 4 || reinterpret_cast<uintptr_t>(scales) % 4)
    return fail(BRQ_ERR_ALIGNMENT, "codes and scales must be 4-byte aligned");
  if (!V && (reinterpret_cast<uintptr_t>(x) % 16 || ldx % 8))
    return fail(BRQ_ERR_ALIGNMENT, "activations need 16-byte aligned rows without a right plan");
  if ((st = check_plan_device(U)) != BRQ_OK) return st;
  if ((st = check_plan_device(V)) != BRQ_OK) return st;
  const QlLayout L = ql_layout(U, V, q, T, m, n);
  if (!ws || ws_bytes < L.total)
    return fail(BRQ_ERR_WORKSPACE, "workspace of %zu bytes < %zu", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // 1. X~ = X M_V^T, in the activation type
  const void* xr = x;
  int64_t ldxr = ldx;
  if (V) {
    st = brq_rotate(right, 0, x, xt, ldx, w + L.xt_off, xt, n, T, n, w + L.rot_off, L.rot_bytes,
                    stream);
    if (st != BRQ_OK) return st;
    xr = w + L.xt_off;
    ldxr = n;
  }
  // 2. the product, split over the input index
  QlArgs a;
  std::memset(&a, 0, sizeof a);
  a.x = xr;
  a.xt = xt;
  a.ldx = ldxr;
  a.T = T;
  a.m = m;
  a.n = n;
  a.codes = codes;
  a.scales = static_cast<const float*>(scales);
  a.bits = q->bits;
  a.group = q->group;
  a.codes_ld = n * q->bits / 8;
  a.scales_ld = n / q->group;
  a.splits = L.splits;
  a.kc = L.kc;
  a.kind = ql_kind(T, m, n, q->bits, q->group, reinterpret_cast<uintptr_t>(codes) % 16 == 0);
  a.tm = ql_kind_tm(a.kind, T, q->bits, q->group);
  a.tn = ql_kind_tn(a.kind, a.tm);
  a.tv = (int)(T < kQlTok * a.tm ? T : kQlTok * a.tm);
  a.part = reinterpret_cast<float*>(w + L.part_off);
  char name[48];
  snprintf(name, sizeof name, "qlinear b%d g%d", q->bits, q->group);
  int tok = prof_begin(name, s);
  hipError_t e = launch_qlinear(a, s);
  prof_end(tok, s);
  if (e != hipSuccess) return hip_fail(e, "quantized linear launch");
  // 3. Y = Z M_U (rows z -> M_U^T z), Z the sum of the parts.  With at most
  // kQlFuseParts parts, when the stage pass takes the inverse rotation and
  // its first launch is the tile kernel, that launch sums the parts as it
  // loads them (the reduction's order) and no separate reduction runs; else
  // the parts are summed into Z first (measured on the 70B down projection:
  // 4 parts at 256 tokens 288.9 -> 281.4 us per call; 32 parts at 16 tokens
  // 73 -> 75 us, the sums then cost the stage more than the launch saved).
  constexpr int kQlFuseParts = 8;
  if (U && L.splits <= kQlFuseParts && fast_paths() && U->mode != BRQ_HADAMARD && sp_rotate_supported(U, 0, T, m)) {
    hipError_t he = hipSuccess;
    st = sp_rotate_stages(U, 0, 1, 0, -1, a.part, BRQ_F32, m, y, yt, ldy, T, m, w + L.rot_off, L.rot_bytes, s,
                          &he, L.splits, T * m);
    if (st != BRQ_ERR_UNSUPPORTED) return stage_fail(st, he, (size_t)T * m * sizeof(float), L.rot_bytes);
  }
  void* zout = U ? static_cast<void*>(w + L.z_off) : y;
  const int zt = U ? (int)BRQ_F32 : yt;
  const int64_t ldz = U ? m : ldy;
  tok = prof_begin("qlinear reduce", s);
  e = launch_ql_reduce(a.part, L.splits, T, m, zout, zt, ldz, s);
  prof_end(tok, s);
  if (e != hipSuccess) return hip_fail(e, "quantized linear reduce launch");
  if (U)
    return brq_rotate_inverse(left, 0, zout, BRQ_F32, m, y, yt, ldy, T, m, w + L.rot_off,
                              L.rot_bytes, stream);
  return BRQ_OK;
}

brq_status brq_lloyd_max_gaussian(int32_t bits, float* centroids) {
  g_last_error.clear();
  if (bits < 1 || bits > 5) return fail(BRQ_ERR_INVALID_ARGUMENT, "bits must be 1..5");
  if (!centroids) return fail(BRQ_ERR_INVALID_ARGUMENT, "centroids is NULL");
  const int L = 1 << bits, h = L / 2;
  // start from the conditional means of equal-mass cells of the half-normal
  std::vector<double> c(h), r, cn(h);
  {
    std::vector<double> edges(h + 1);
    edges[0] = 0.0;
    for (int k = 1; k < h; ++k) {
      // invert the half-normal CDF by bisection
      const double target = (double)k / h;
      double lo = 0, hi = 40;
      for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (lo + hi);
        (1.0 - 2.0 * upper_tail(mid) < target ? lo : hi) = mid;
      }
      edges[k] = 0.5 * (lo + hi);
    }
    edges[h] = INFINITY;
    for (int k = 0; k < h; ++k) {
      const double a = edges[k], b = edges[k + 1];
      const double mass = upper_tail(a) - (std::isinf(b) ? 0.0 : upper_tail(b));
      c[k] = (npdf(a) - (std::isinf(b) ? 0.0 : npdf(b))) / mass;
    }
  }
  // fixed-point iteration of the two optimality conditions ...
  for (int it = 0; it < 2000; ++it) {
    lm_residual(c, r);
    for (int k = 0; k < h; ++k) c[k] -= r[k];
  }
  // ... then Newton steps with a finite-difference Jacobian
  for (int it = 0; it < 50; ++it) {
    lm_residual(c, r);
    double err = 0;
    for (double v : r) err = std::max(err, std::fabs(v));
    if (err < 1e-14) break;
    std::vector<double> J(h * h), rp;
    for (int j = 0; j < h; ++j) {
      std::vector<double> cp = c;
      const double step = 1e-7 * std::max(1.0, std::fabs(c[j]));
      cp[j] += step;
      lm_residual(cp, rp);
      for (int i = 0; i < h; ++i) J[i * h + j] = (rp[i] - r[i]) / step;
    }
    // solve J dx = r (Gaussian elimination with partial pivoting)
    std::vector<double> bvec = r;
    for (int col = 0; col < h; ++col) {
      int piv = col;
      for (int i = col + 1; i < h; ++i)
        if (std::fabs(J[i * h + col]) > std::fabs(J[piv * h + col])) piv = i;
      if (piv != col) {
        for (int k = 0; k < h; ++k) std::swap(J[col * h + k], J[piv * h + k]);
        std::swap(bvec[col], bvec[piv]);
      }
      for (int i = col + 1; i < h; ++i) {
        const double f = J[i * h + col] / J[col * h + col];
        for (int k = col; k < h; ++k) J[i * h + k] -= f * J[col * h + k];
        bvec[i] -= f * bvec[col];
      }
    }
    for (int i = h - 1; i >= 0; --i) {
      double acc = bvec[i];
      for (int k = i + 1; k < h; ++k) acc -= J[i * h + k] * cn[k];
      cn[i] = acc / J[i * h + i];
    }
    for (int k = 0; k < h; ++k) c[k] -= cn[k];
  }
  lm_residual(c, r);
  double err = 0;
  for (double v : r) err = std::max(err, std::fabs(v));
  if (!(err < 1e-12)) return fail(BRQ_ERR_UNSUPPORTED, "Lloyd-Max did not converge (%g)", err);
  for (int k = 0; k < h; ++k) {
    centroids[h + k] = (float)c[k];
    centroids[h - 1 - k] = (float)-c[k];
  }
  return BRQ_OK;
}

// ---- ORP GEO quantizer ----------------------------------------------------------

namespace {

brq_status check_orp(const brq_orp* q, int64_t n) {
  if (!q) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL quantizer");
  if (q->bits < 2 || q->bits > 5) return fail(BRQ_ERR_UNSUPPORTED, "bits must be 2..5");
  if (q->group != 64 && q->group != 128 && q->group != 256 && q->group != 512)
    return fail(BRQ_ERR_UNSUPPORTED, "group must be 64, 128, 256 or 512");
  if (!is_pow2(q->stride) || 2 * q->stride > q->group)
    return fail(BRQ_ERR_INVALID_ARGUMENT, "stride must be a power of two with 2*stride <= group");
  if (n % q->group) return fail(BRQ_ERR_INVALID_ARGUMENT, "group %d does not divide n", q->group);
  return BRQ_OK;
}

brq_status orp_outputs_ok(const uint8_t* codes, const uint8_t* signs, const float* coef) {
  if (!codes || !signs || !coef) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 4 || reinterpret_cast<uintptr_t>(coef) % 8)
    return fail(BRQ_ERR_ALIGNMENT, "codes must be 4-byte and coef 8-byte aligned");
  return BRQ_OK;
}

size_t dtype_bytes(int t) { return t == BRQ_F32 ? 4 : 2; }

void orp_strides(OrpArgs& a) {
  a.lg_group = 0;
  while ((1 << a.lg_group) < a.group) ++a.lg_group;
  a.lg_stride = 0;
  while ((1 << a.lg_stride) < a.stride) ++a.lg_stride;
  a.codes_ld = a.n * a.bits / 8;
  a.signs_ld = a.n / 16;
  a.coef_ld = 2 * (a.n / a.group);
}

}  // namespace

brq_status brq_orp_geo_quantize(const void* w, int32_t wt, int64_t m, int64_t n, int64_t ldw,
                                const float* smooth, const brq_orp* q, uint8_t* codes,
                                uint8_t* signs, float* coef, void* stream) {
  g_last_error.clear();
  if (!valid_dtype(wt)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad input dtype");
  if (m < 0 || n < 0 || ldw < n) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad shape or leading dimension");
  brq_status st = check_orp(q, n);
  if (st != BRQ_OK) return st;
  if (n >= ((int64_t)1 << 31)) return fail(BRQ_ERR_UNSUPPORTED, "rows longer than 2^31 elements");
  if (m == 0 || n == 0) return BRQ_OK;
  if (!w) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if ((st = orp_outputs_ok(codes, signs, coef)) != BRQ_OK) return st;
  if (reinterpret_cast<uintptr_t>(w) % 16 || (ldw * dtype_bytes(wt)) % 16)
    return fail(BRQ_ERR_ALIGNMENT, "input rows must be 16-byte aligned");
  if (smooth && reinterpret_cast<uintptr_t>(smooth) % 16)
    return fail(BRQ_ERR_ALIGNMENT, "the smoothing vector must be 16-byte aligned");
  OrpArgs a;
  std::memset(&a, 0, sizeof a);
  a.w = w;
  a.wt = wt;
  a.ldw = ldw;
  a.smooth = smooth;
  a.m = m;
  a.n = n;
  a.bits = q->bits;
  a.group = q->group;
  a.stride = q->stride;
  a.chunks = (n + kOrpChunk - 1) / kOrpChunk;
  orp_strides(a);
  a.codes = codes;
  a.signs = signs;
  a.coef = coef;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char name[48];
  snprintf(name, sizeof name, "orp geo quant b%d g%d S%d", q->bits, q->group, q->stride);
  const int tok = prof_begin(name, s);
  const hipError_t e = launch_orp_quant(a, s);
  prof_end(tok, s);
  if (e != hipSuccess) return hip_fail(e, "ORP quantizer launch");
  return BRQ_OK;
}

brq_status brq_orp_geo_dequant(const uint8_t* codes, const uint8_t* signs, const float* coef,
                               const brq_orp* q, int64_t m, int64_t n, void* out, int32_t ot,
                               int64_t ldo, void* stream) {
  g_last_error.clear();
  if (!valid_dtype(ot)) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad output dtype");
  if (m < 0 || n < 0 || ldo < n) return fail(BRQ_ERR_INVALID_ARGUMENT, "bad shape or leading dimension");
  brq_status st = check_orp(q, n);
  if (st != BRQ_OK) return st;
  if (n >= ((int64_t)1 << 31)) return fail(BRQ_ERR_UNSUPPORTED, "rows longer than 2^31 elements");
  if (m == 0 || n == 0) return BRQ_OK;
  if (!out) return fail(BRQ_ERR_INVALID_ARGUMENT, "NULL data pointer");
  if ((st = orp_outputs_ok(codes, signs, coef)) != BRQ_OK) return st;
  if (reinterpret_cast<uintptr_t>(out) % 16 || (ldo * dtype_bytes(ot)) % 16)
    return fail(BRQ_ERR_ALIGNMENT, "output rows must be 16-byte aligned");
  OrpArgs a;
  std::memset(&a, 0, sizeof a);
  a.m = m;
  a.n = n;
  a.bits = q->bits;
  a.group = q->group;
  a.stride = q->stride;
  a.chunks = (n + kOrpChunk - 1) / kOrpChunk;
  orp_strides(a);
  a.codes = const_cast<uint8_t*>(codes);
  a.signs = const_cast<uint8_t*>(signs);
  a.coef = const_cast<float*>(coef);
  a.out = out;
  a.ot = ot;
  a.ldo = ldo;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char name[48];
  snprintf(name, sizeof name, "orp geo dequant b%d g%d S%d", q->bits, q->group, q->stride);
  const int tok = prof_begin(name, s);
  const hipError_t e = launch_orp_dequant(a, s);
  prof_end(tok, s);
  if (e != hipSuccess) return hip_fail(e, "ORP dequantizer launch");
  return BRQ_OK;
}

}  // extern "C"
