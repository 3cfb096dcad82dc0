// Host side of the two-sided fast path: plan preparation, the coverage test
// and the launch of its two kernels.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fused.h"

namespace brq {

int prof_begin(const char* name, hipStream_t s);
void prof_end(int token, hipStream_t s);

namespace {

// Radix of stage 0 when the plan fits the fast path as (b0, 16, 16), else 0.
// A Hadamard plan of any power-of-two radix schedule is the Sylvester matrix
// H_d / sqrt(d) = (H_b0 / sqrt(b0)) x (H_16 / 4) x (H_16 / 4) in natural order,
// so for d = 256 b0 it is taken as that three-stage schedule.
int fused_b0(const Plan& p) {
  if (p.mode == BRQ_HADAMARD) {
    const int b0 = p.d / 256;
    return p.d % 256 == 0 && b0 >= 2 && b0 <= 64 && (b0 & (b0 - 1)) == 0 ? b0 : 0;
  }
  const bool fits = p.nst == 3 && p.radix[1] == 16 && p.radix[2] == 16 && p.radix[0] >= 2 &&
                    p.radix[0] <= 64;
  return fits ? p.radix[0] : 0;
}

// Sylvester Hadamard block H_b / sqrt(b), row-major, H[j][k] = (-1)^popcount(j & k).
void hadamard_block(int b, float* out) {
  const float s = 1.0f / std::sqrt((float)b);
  for (int j = 0; j < b; ++j)
    for (int k = 0; k < b; ++k) out[j * b + k] = (__builtin_popcount(j & k) & 1) ? -s : s;
}

}  // namespace

// Stage-0 blocks for the fast path: zero-padded to 16*nb, with the plan's
// signs folded in.  M = ... B_0 D, and the members of stage-0 group c are
// i = k*S_0 + c (S_0 = 256), so (B_0 D) restricted to group c is
// B_{0,c} diag(s[k*256 + c]): column k of the block times that sign.
hipError_t fused_prepare(Plan& p, const float* host_blocks, const int8_t* host_signs) {
  const int b0 = fused_b0(p);
  if (!b0) return hipSuccess;
  const int nb = (b0 + 15) / 16;
  const int np = 16 * nb;
  const int S0 = 256;  // stride of stage 0 in the (b0, 16, 16) schedule
  const bool shared_src = p.mode != BRQ_PER_GROUP;
  const bool per_group = !shared_src || host_signs;
  const int ng0 = per_group ? S0 : 1;
  std::vector<float> src;
  if (p.mode == BRQ_HADAMARD) {
    src.resize((size_t)b0 * b0);
    hadamard_block(b0, src.data());
  }
  const float* g0 = p.mode == BRQ_HADAMARD ? src.data() : host_blocks + p.blk_off[0];
  std::vector<float> pad((size_t)ng0 * np * np, 0.f);
  for (int g = 0; g < ng0; ++g) {
    const float* blk = g0 + (shared_src ? 0 : (size_t)g * b0 * b0);
    for (int j = 0; j < b0; ++j)
      for (int k = 0; k < b0; ++k) {
        const float sg = host_signs ? (float)host_signs[(size_t)k * S0 + g] : 1.0f;
        pad[((size_t)g * np + j) * np + k] = blk[j * b0 + k] * sg;
      }
  }
  // the same blocks in pass A's fragment order: lane (lr, lg) of output tile
  // nt reads the 4 nb steps V[16 nt + lr][4 s + lg] as consecutive floats
  std::vector<float> frag(pad.size());
  for (int g = 0; g < ng0; ++g)
    for (int nt = 0; nt < nb; ++nt)
      for (int lr = 0; lr < 16; ++lr)
        for (int lg = 0; lg < 4; ++lg)
          for (int st = 0; st < 4 * nb; ++st)
            frag[(size_t)g * np * np + fa_vfrag(nb, nt, lr, lg, st)] =
                pad[((size_t)g * np + 16 * nt + lr) * np + 4 * st + lg];
  hipError_t e = rt_malloc((void**)&p.fz0, pad.size() * sizeof(float));
  if (e == hipSuccess) e = rt_copy_to_device(p.fz0, pad.data(), pad.size() * sizeof(float));
  if (e == hipSuccess) e = rt_malloc((void**)&p.fz0f, frag.size() * sizeof(float));
  if (e == hipSuccess) e = rt_copy_to_device(p.fz0f, frag.data(), frag.size() * sizeof(float));
  if (e != hipSuccess) return e;
  p.fz_b0 = b0;
  p.fz_nb = nb;
  p.fz_gs0 = per_group ? (int64_t)np * np : 0;
  if (p.mode == BRQ_HADAMARD) {
    std::vector<float> h16(256);
    hadamard_block(16, h16.data());
    e = rt_malloc((void**)&p.fz_had, 256 * sizeof(float));
    if (e == hipSuccess) e = rt_copy_to_device(p.fz_had, h16.data(), 256 * sizeof(float));
    if (e != hipSuccess) return e;
    p.fz1 = p.fz_had;
    p.fz2 = p.fz_had;
    p.fz_gs1 = p.fz_gs2 = 0;
  } else {
    p.fz1 = p.blk + p.blk_off[1];
    p.fz2 = p.blk + p.blk_off[2];
    p.fz_gs1 = p.fz_gs2 = shared_src ? 0 : 256;
  }
  p.fz_ok = 1;
  return hipSuccess;
}

namespace {

// Persistent pass B: one workgroup per compute unit (its LDS use allows no
// more), capped by the tile count.
int fused_b_grid(const FusedBArgs& b) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (rt_get_device(&dev) != hipSuccess || rt_cu_count(dev, &cus) != hipSuccess || cus < 1)
      cus = 256;
  }
  const int64_t nt = fb_nwg(b);
  return (int)(nt < cus ? nt : cus);
}

const char* check_b(const FusedBArgs& b);

// Host check of what the two kernels' index arithmetic relies on.
const char* check_fused(const FusedAArgs& a, const FusedBArgs& b) {
  if (a.bv < 2 || a.bv > 64 || a.nb != (a.bv + 15) / 16) return "V_0 radix";
  if (a.m != 4096 || a.dv != a.bv * 256 || (int64_t)a.nchunk * a.dv != a.n) return "shape";
  if (fa_nwg(a) % 8) return "pass A grid";
  for (int i = 0; i < 16 * a.bv; ++i)  // the multiply-shift quotient is exact where used
    if (fa_div_bv(a, i) != i / a.bv) return "division multiplier";
  if (fa_lds_bytes(fa_geom(a.wt, a.nb, a.bv)) > 160 * 1024) return "pass A LDS";
  // pass A addresses a lane's input and output as 32-bit byte offsets from a
  // per-chunk base
  if ((int64_t)a.m * a.ldw * fa_esz(a.wt) >= (int64_t(1) << 31) ||
      (int64_t)a.m * a.n * 4 >= (int64_t(1) << 31))
    return "32-bit offsets";
  if (!a.w || !a.ws || !a.u0 || !a.v0f) return "pass A pointers";
  if (a.u0_gs && a.u0_n < 256 * a.u0_gs) return "U_0 extent";
  if (a.v0_gs && a.v0_n < 256 * a.v0_gs) return "V_0 extent";
  if (a.u0_n < 256 || a.v0_n < 256 * a.nb * a.nb) return "block extent";
  if (b.bv != a.bv || b.nchunk != a.nchunk || b.dv != a.dv || b.m != a.m || b.n != a.n)
    return "pass B shape";
  return check_b(b);
}

// Host check of pass B alone.
const char* check_b(const FusedBArgs& b) {
  if (b.m < 256 || b.m % 256 || b.nrb != b.m / 256 || b.dv != b.bv * 256 || b.bv < 1 ||
      (int64_t)b.nchunk * b.dv != b.n)
    return "pass B shape";
  if ((int64_t)b.m * b.n * 4 >= (int64_t(1) << 40)) return "pass B extent";
  if (!b.ws || !b.u1 || !b.u2 || !b.v1 || !b.v2 || !b.codes || !b.scales) return "pass B pointers";
  if (b.u1_gs && b.u1_n < (int64_t)b.nrb * 16 * b.u1_gs) return "U_1 extent";
  if (b.u2_gs && b.u2_n < (int64_t)b.nrb * 16 * b.u2_gs) return "U_2 extent";
  if (b.v1_gs && b.v1_n < (int64_t)b.bv * 16 * b.v1_gs) return "V_1 extent";
  if (b.v2_gs && b.v2_n < (int64_t)b.bv * 16 * b.v2_gs) return "V_2 extent";
  if (b.group != 64 && b.group != 128) return "group";
  if (b.bits < 2 || b.bits > 5 || b.nlev != (1 << b.bits)) return "bits";
  if (b.codes_ld * 8 != b.n * b.bits || b.codes_ld % 4 || b.scales_ld * b.group != b.n)
    return "code layout";
  return nullptr;
}

void fill_quant_b(FusedBArgs& b, const brq_quant* q, int64_t n) {
  b.qkind = q->kind;
  b.bits = q->bits;
  b.group = q->group;
  b.nlev = 1 << q->bits;
  b.h = (float)((b.nlev - 1) * 0.5);
  b.sqrt_g = std::sqrt((float)q->group);
  for (int i = 0; i + 1 < b.nlev; ++i)
    b.tau[i] = q->kind == BRQ_CODEBOOK_NORM ? (q->codebook[i] + q->codebook[i + 1]) * 0.5f : 0.f;
  b.codes_ld = n * q->bits / 8;
  b.scales_ld = n / q->group;
}

}  // namespace

void fused_release(Plan& p) {
  rt_free(p.fz0);
  rt_free(p.fz0f);
  rt_free(p.fz_had);
  p.fz0 = p.fz0f = p.fz_had = nullptr;
  p.fz_ok = 0;
  p.fz_b0 = 0;
}

bool fused_rotate_supported(const Plan*, const Plan*, int, int, int64_t, int64_t, int64_t, int64_t,
                            const void*, const void*) {
  return false;
}

hipError_t fused_rotate(const Plan*, const Plan*, const void*, int, int64_t, void*, int, int64_t,
                        int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

// Two-sided, left (16,16,16) over all rows, right (b0,16,16) on every d-chunk
// of a row, 16-byte aligned rows, quantizer groups of 64 or 128 columns with
// whole 32-bit code words per group and per row.
bool fused_rqp_supported(const Plan* U, const Plan* V, int wt, int64_t m, int64_t n, int64_t ldw,
                         const void* w, const brq_quant* q) {
  if (!U || !V || !U->fz_ok || !V->fz_ok) return false;
  if (U->fz_b0 != 16 || U->d != m || n % V->d) return false;
  if (q->group != 64 && q->group != 128) return false;
  if ((n * q->bits) % 32) return false;
  const int elem = wt == BRQ_F32 ? 4 : 2;
  if ((ldw * elem) % 16 || reinterpret_cast<uintptr_t>(w) % 16) return false;
  return true;
}

brq_status fused_rqp(const Plan* U, const Plan* V, const void* w, int wt, int64_t m, int64_t n,
                     int64_t ldw, const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  const size_t need = (size_t)m * n * sizeof(float);
  if (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 16) return BRQ_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(codes) % 4 || reinterpret_cast<uintptr_t>(scales) % 4)
    return BRQ_ERR_UNSUPPORTED;

  FusedAArgs a;
  std::memset(&a, 0, sizeof a);
  a.w = w;
  a.wt = wt;
  a.ldw = ldw;
  a.ws = static_cast<float*>(ws);
  a.m = m;
  a.n = n;
  a.bv = V->fz_b0;
  a.nb = V->fz_nb;
  a.dv = V->d;
  a.nchunk = (int)(n / V->d);
  a.u0 = U->fz0;  // radix 16: the padded layout is the 16 x 16 block itself
  a.u0_gs = U->fz_gs0;
  a.v0f = V->fz0f;
  a.v0_gs = V->fz_gs0;
  a.bv_magic = (uint32_t)((1ull << 32) / (uint64_t)a.bv + 1);

  FusedBArgs b;
  std::memset(&b, 0, sizeof b);
  b.ws = a.ws;
  b.m = m;
  b.n = n;
  b.nrb = (int)(m / 256);
  b.bv = a.bv;
  b.nchunk = a.nchunk;
  b.dv = a.dv;
  b.u1 = U->fz1;
  b.u1_gs = U->fz_gs1;
  b.u2 = U->fz2;
  b.u2_gs = U->fz_gs2;
  b.v1 = V->fz1;
  b.v1_gs = V->fz_gs1;
  b.v2 = V->fz2;
  b.v2_gs = V->fz_gs2;
  fill_quant_b(b, q, n);
  b.codes = codes;
  b.scales = scales;
  const int64_t u16 = U->mode == BRQ_PER_GROUP ? (int64_t)(U->d / 16) * 256 : 256;
  const int64_t v16 = V->mode == BRQ_PER_GROUP ? (int64_t)(V->d / 16) * 256 : 256;
  a.u0_n = (U->fz_gs0 ? 256 : 1) * 256;
  a.v0_n = (V->fz_gs0 ? 256 : 1) * 256 * a.nb * a.nb;
  b.u1_n = b.u2_n = u16;
  b.v1_n = b.v2_n = v16;
  if (check_fused(a, b)) return BRQ_ERR_UNSUPPORTED;

  char name[96];
  snprintf(name, sizeof name, "fusedA U0(16) V0(%d)", a.bv);
  int tok = prof_begin(name, s);
  hipError_t e = launch_fused_a(a, s);
  prof_end(tok, s);
  if (e != hipSuccess) return BRQ_ERR_HIP;
  snprintf(name, sizeof name, "fusedB U(16,16) V(16,16) quant b%d g%d", q->bits, q->group);
  tok = prof_begin(name, s);
  e = launch_fused_b(b, fused_b_grid(b), s);
  prof_end(tok, s);
  return e == hipSuccess ? BRQ_OK : BRQ_ERR_HIP;
}

namespace {
// The last two stages of a dense plan are radix 16 (and the plan has more).
bool dense_tail16(const Plan* p) {
  return p && p->mode != BRQ_HADAMARD && p->nst >= 3 && p->radix[p->nst - 2] == 16 &&
         p->radix[p->nst - 1] == 16 && p->d % 256 == 0;
}
}  // namespace

bool fused_tail_supported(const Plan* U, const Plan* V, int64_t m, int64_t n, const brq_quant* q) {
  if (!dense_tail16(U) || !dense_tail16(V) || U->d != m || n % V->d) return false;
  if (q->group != 64 && q->group != 128) return false;
  return (n * q->bits) % 32 == 0;
}

brq_status fused_tail_rqp(const Plan* U, const Plan* V, const float* ws, int64_t m, int64_t n,
                          const brq_quant* q, uint8_t* codes, void* scales, hipStream_t s) {
  if (reinterpret_cast<uintptr_t>(ws) % 16 || reinterpret_cast<uintptr_t>(codes) % 4 ||
      reinterpret_cast<uintptr_t>(scales) % 4)
    return BRQ_ERR_UNSUPPORTED;
  FusedBArgs b;
  std::memset(&b, 0, sizeof b);
  b.ws = ws;
  b.m = m;
  b.n = n;
  b.nrb = (int)(m / 256);
  b.bv = V->d / 256;
  b.dv = V->d;
  b.nchunk = (int)(n / V->d);
  // stage t's per-group blocks: group c at c * 256 floats (shared: one block)
  const bool ug = U->mode == BRQ_PER_GROUP, vg = V->mode == BRQ_PER_GROUP;
  b.u1 = U->blk + U->blk_off[U->nst - 2];
  b.u2 = U->blk + U->blk_off[U->nst - 1];
  b.v1 = V->blk + V->blk_off[V->nst - 2];
  b.v2 = V->blk + V->blk_off[V->nst - 1];
  b.u1_gs = b.u2_gs = ug ? 256 : 0;
  b.v1_gs = b.v2_gs = vg ? 256 : 0;
  b.u1_n = b.u2_n = ug ? (int64_t)(U->d / 16) * 256 : 256;
  b.v1_n = b.v2_n = vg ? (int64_t)(V->d / 16) * 256 : 256;
  fill_quant_b(b, q, n);
  b.codes = codes;
  b.scales = scales;
  if (check_b(b)) return BRQ_ERR_UNSUPPORTED;
  char name[96];
  snprintf(name, sizeof name, "fusedB U(16,16) V(16,16) quant b%d g%d", q->bits, q->group);
  const int tok = prof_begin(name, s);
  const hipError_t e = launch_fused_b(b, fused_b_grid(b), s);
  prof_end(tok, s);
  return e == hipSuccess ? BRQ_OK : BRQ_ERR_HIP;
}

}  // namespace brq
