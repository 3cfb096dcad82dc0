// Host side of the row Hadamard path: which calls it takes, argument set-up
// and launch.
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "rowhad.h"

namespace brq {

int prof_begin(const char* name, hipStream_t s);
void prof_end(int token, hipStream_t s);

namespace {

int log2i(int d) {
  int l = 0;
  while ((1 << l) < d) ++l;
  return l;
}

int elem_size(int t) { return t == BRQ_F32 ? 4 : 2; }

// 16-element runs of a row are 16-byte aligned.
bool rows_aligned(const void* p, int t, int64_t ld) {
  return reinterpret_cast<uintptr_t>(p) % 16 == 0 && (ld * elem_size(t)) % 16 == 0;
}

void fill_common(RhArgs& a, const Plan* p, int64_t rows, int64_t n) {
  std::memset(&a, 0, sizeof a);
  a.log2d = log2i(p->d);
  a.rows = rows;
  a.n = n;
  a.cpr = n / p->d;
  a.nchunks = rows * a.cpr;
  a.signs = p->signs;
  a.signs_s = p->signs_s;
  a.scale = 1.0f / std::sqrt((float)p->d);
}

void fill_quant(RhArgs& a, const brq_quant* q, int64_t n) {
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
  a.bin_s = a.bin_off = 0.f;
  if (q->kind != BRQ_CODEBOOK_NORM) return;
  // Find a scaling that puts each threshold in its own bin, away from bin
  // edges, in the kernel's fp32 arithmetic.
  const int nt = a.nlev - 1;
  const float lo = a.tau[0], hi = a.tau[nt - 1];
  for (int tries = 0; tries < 64; ++tries) {
    const float span = hi - lo;
    const float s = (float)(kRhBins - 8) / (span > 0.f ? span : 1.f) / (1.f + 0.03125f * tries);
    const float off = 4.f - lo * s + 0.37f * (float)tries;
    bool ok = true;
    int prev = -1;
    for (int i = 0; i < nt && ok; ++i) {
      const float u = std::fma(a.tau[i], s, off);
      const int b = (int)std::floor(u);
      const float f = u - (float)b;
      ok = b >= 1 && b < kRhBins - 1 && b > prev && f > 1.f / 64 && f < 1.f - 1.f / 64 &&
           rh_bin(u) == b;
      prev = b;
    }
    if (ok) {
      a.bin_s = s;
      a.bin_off = off;
      for (int i = 0; i < nt; ++i) a.tbin[i] = rh_bin(std::fma(a.tau[i], s, off));
      for (int b = 0; b < kRhBins; ++b) {
        float tin = INFINITY;
        int cnt = 0;
        for (int i = 0; i < nt; ++i) {
          cnt += a.tbin[i] < b ? 1 : 0;
          if (a.tbin[i] == b) tin = a.tau[i];
        }
        // the threshold in the bins' coordinate, as the kernel compares it
        float cbits;
        std::memcpy(&cbits, &cnt, sizeof cbits);
        a.bintab[b] = make_float2(tin == INFINITY ? INFINITY : std::fma(tin, s, off), cbits);
      }
      return;
    }
  }
}

brq_status launch(const RhArgs& a, const char* what, hipStream_t s) {
  const int tok = prof_begin(what, s);
  const hipError_t e = launch_rowhad(a, s);
  prof_end(tok, s);
  return e == hipSuccess ? BRQ_OK : BRQ_ERR_HIP;
}

}  // namespace

bool rh_rotate_supported(const Plan* p, int side, int xt, int yt, int64_t rows, int64_t cols,
                         int64_t ldx, int64_t ldy, const void* x, const void* y) {
  if (side != 0 || !rh_plan_ok(p) || cols % p->d) return false;
  if (x == y) return false;  // in place goes through the tile pass
  if (rows * (cols / p->d) > kRhMaxChunks) return false;
  return rows > 0 && rows_aligned(x, xt, ldx) && rows_aligned(y, yt, ldy);
}

brq_status rh_rotate(const Plan* p, int inverse, const void* x, int xt, int64_t ldx, void* y,
                     int yt, int64_t ldy, int64_t rows, int64_t cols, hipStream_t s) {
  RhArgs a;
  fill_common(a, p, rows, cols);
  a.mode = RH_ROTATE;
  a.x = x;
  a.xt = xt;
  a.ldx = ldx;
  a.y = y;
  a.yt = yt;
  a.ldy = ldy;
  a.inverse = inverse;
  char name[64];
  snprintf(name, sizeof name, "rowhad R%s(H%d)", inverse ? "^T" : "", p->d);
  return launch(a, name, s);
}

bool rh_quant_supported(const Plan* U, const Plan* V, int wt, int64_t m, int64_t n, int64_t ldw,
                        const void* w, const brq_quant* q) {
  if (U || !rh_plan_ok(V) || n % V->d) return false;
  if (m * (n / V->d) > kRhMaxChunks) return false;
  // a quantizer group lies inside one workgroup's 4096 elements of a row
  if (q->group > 1024 || kRhTile % q->group) return false;
  return rows_aligned(w, wt, ldw);
}

brq_status rh_rqp(const Plan* V, const void* w, int wt, int64_t m, int64_t n, int64_t ldw,
                  const brq_quant* q, uint8_t* codes, void* scales, hipStream_t s) {
  if (reinterpret_cast<uintptr_t>(codes) % 4 || reinterpret_cast<uintptr_t>(scales) % 4)
    return BRQ_ERR_UNSUPPORTED;
  RhArgs a;
  fill_common(a, V, m, n);
  fill_quant(a, q, n);
  a.mode = RH_QUANT;
  a.x = w;
  a.xt = wt;
  a.ldx = ldw;
  a.codes = codes;
  a.scales = scales;
  char name[64];
  snprintf(name, sizeof name, "rowhad R(H%d) quant b%d g%d", V->d, q->bits, q->group);
  return launch(a, name, s);
}

brq_status rh_quant_only(const void* w, int wt, int64_t m, int64_t n, int64_t ldw,
                         const brq_quant* q, uint8_t* codes, void* scales, hipStream_t s) {
  if (n % 16 || q->group > 1024 || kRhTile % q->group || !rows_aligned(w, wt, ldw) ||
      m * (n / 16) > kRhMaxChunks || reinterpret_cast<uintptr_t>(codes) % 4 ||
      reinterpret_cast<uintptr_t>(scales) % 4)
    return BRQ_ERR_UNSUPPORTED;
  Plan id;  // d = 16, no blocks or signs: only the shape of the row split
  id.d = 16;
  RhArgs a;
  fill_common(a, &id, m, n);
  fill_quant(a, q, n);
  a.mode = RH_QUANT;
  a.identity = 1;
  a.scale = 1.0f;
  a.x = w;
  a.xt = wt;
  a.ldx = ldw;
  a.codes = codes;
  a.scales = scales;
  char name[64];
  snprintf(name, sizeof name, "rowhad quant b%d g%d", q->bits, q->group);
  return launch(a, name, s);
}

brq_status rh_dequant(const Plan* V, const uint8_t* codes, const void* scales, const brq_quant* q,
                      int64_t m, int64_t n, void* out, int ot, int64_t ldo, hipStream_t s) {
  if (reinterpret_cast<uintptr_t>(codes) % 4 || reinterpret_cast<uintptr_t>(scales) % 4 ||
      !rows_aligned(out, ot, ldo) || m * (n / V->d) > kRhMaxChunks)
    return BRQ_ERR_UNSUPPORTED;
  RhArgs a;
  fill_common(a, V, m, n);
  fill_quant(a, q, n);
  a.mode = RH_DEQUANT;
  a.inverse = 1;
  a.in_codes = codes;
  a.in_scales = scales;
  a.y = out;
  a.yt = ot;
  a.ldy = ldo;
  char name[64];
  snprintf(name, sizeof name, "rowhad dequant R^T(H%d) b%d g%d", V->d, q->bits, q->group);
  return launch(a, name, s);
}

brq_status rh_requant(const Plan* V, const uint8_t* codes, const void* scales, const brq_quant* q_in,
                      int64_t m, int64_t n, const brq_quant* q_out, uint8_t* codes_out,
                      void* scales_out, hipStream_t s) {
  if (!rh_plan_ok(V) || V->d < 64 || V->d > 256 || n % V->d || q_out->kind != BRQ_ABSMAX ||
      q_out->group > 1024 || kRhTile % q_out->group || m * (n / V->d) > kRhMaxChunks ||
      reinterpret_cast<uintptr_t>(codes) % 4 || reinterpret_cast<uintptr_t>(scales) % 4 ||
      reinterpret_cast<uintptr_t>(codes_out) % 4 || reinterpret_cast<uintptr_t>(scales_out) % 4)
    return BRQ_ERR_UNSUPPORTED;
  RhArgs a;
  fill_common(a, V, m, n);
  fill_quant(a, q_in, n);
  a.mode = RH_REQUANT;
  a.inverse = 1;
  a.in_codes = codes;
  a.in_scales = scales;
  a.bits2 = q_out->bits;
  a.group2 = q_out->group;
  a.h2 = (float)(((1 << q_out->bits) - 1) * 0.5);
  a.codes_ld2 = n * q_out->bits / 8;
  a.scales_ld2 = n / q_out->group;
  a.codes = codes_out;
  a.scales = scales_out;
  char name[80];
  snprintf(name, sizeof name, "rowhad requant R^T(H%d) b%d g%d -> absmax b%d g%d", V->d, q_in->bits,
           q_in->group, q_out->bits, q_out->group);
  return launch(a, name, s);
}

}  // namespace brq
