// Host side of the two-sided fast path: plan preparation, the coverage test
// and the launch of its two kernels.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fused.h"
#include "stage.h"

namespace brq {

int prof_begin(const char* name, hipStream_t s);
void prof_end(int token, hipStream_t s);

namespace {

// Radix of stage 0 when the plan fits pass A and pass B, else 0: stage 0 of
// radix at most 64, then any stages (stage passes apply them between the two
// passes), then two of radix 16.  A Hadamard plan of any power-of-two radix
// schedule is the Sylvester matrix H_d / sqrt(d) = (H_b0 / sqrt(b0)) x
// (H_16 / 4) x (H_16 / 4) in natural order, so for d = 256 b0 it is taken as
// that three-stage schedule.
int fused_b0(const Plan& p) {
  if (p.mode == BRQ_HADAMARD) {
    const int b0 = p.d / 256;
    return p.d % 256 == 0 && b0 >= 2 && b0 <= 64 && (b0 & (b0 - 1)) == 0 ? b0 : 0;
  }
  const bool fits = p.nst >= 3 && p.radix[p.nst - 2] == 16 && p.radix[p.nst - 1] == 16 &&
                    p.radix[0] >= 2 && p.radix[0] <= 64 && p.stride[0] % 256 == 0;
  return fits ? p.radix[0] : 0;
}

// Stride of that stage 0.
int fused_s0(const Plan& p) { return p.mode == BRQ_HADAMARD ? 256 : p.stride[0]; }

// Stages between stage 0 and the last two (none for Hadamard plans, which
// run as (b0, 16, 16)).
int mid_stages(const Plan& p) { return p.mode == BRQ_HADAMARD ? 0 : p.nst - 3; }

// Sylvester Hadamard block H_b / sqrt(b), row-major, H[j][k] = (-1)^popcount(j & k).
void hadamard_block(int b, float* out) {
  const float s = 1.0f / std::sqrt((float)b);
  for (int j = 0; j < b; ++j)
    for (int k = 0; k < b; ++k) out[j * b + k] = (__builtin_popcount(j & k) & 1) ? -s : s;
}

// Split-f16 copies of pass B's blocks: the last two stages of a plan whose
// last two radices are 16 (Hadamard plans of the fast path: H_16 / 4, shared).
// Each entry x becomes hi = f16(x) and lo = f16(x - hi), both rounded to
// nearest even.  Returns hipSuccess with p.fzh unset when the plan does not
// qualify or a block row has norm above 1 + 1e-3 (pass B's range bound).
hipError_t prepare_split16(Plan& p, const float* host_blocks) {
  std::vector<float> had;
  int64_t groups = 0;
  const float* st[2] = {nullptr, nullptr};
  if (p.mode == BRQ_HADAMARD) {
    if (!fused_b0(p)) return hipSuccess;
    had.resize(256);
    hadamard_block(16, had.data());
    st[0] = st[1] = had.data();
    groups = 1;
  } else {
    if (p.nst < 3 || p.radix[p.nst - 2] != 16 || p.radix[p.nst - 1] != 16 || p.d % 256) return hipSuccess;
    groups = p.mode == BRQ_PER_GROUP ? p.d / 16 : 1;
    st[0] = host_blocks + p.blk_off[p.nst - 2];
    st[1] = host_blocks + p.blk_off[p.nst - 1];
  }
  const int64_t per = groups * kFbBlockHalves;
  std::vector<uint16_t> out((size_t)(2 * per));
  bool exact = true;
  for (int s = 0; s < 2; ++s)
    for (int64_t g = 0; g < groups; ++g) {
      const float* blk = st[s] + g * 256;
      for (int j = 0; j < 16; ++j) {
        double nrm = 0;
        for (int k = 0; k < 16; ++k) nrm += (double)blk[j * 16 + k] * blk[j * 16 + k];
        if (!(nrm <= 1.002)) return hipSuccess;  // (1 + 1e-3)^2, and not NaN
        for (int k = 0; k < 16; ++k) {
          const float x = blk[j * 16 + k];
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)(x - (float)hi);
          if ((float)lo != 0.0f) exact = false;
          uint16_t* e = out.data() + s * per + g * kFbBlockHalves + fb_hentry(j, k / 4);
          e[k % 4] = __builtin_bit_cast(uint16_t, hi);
          e[4 + k % 4] = __builtin_bit_cast(uint16_t, lo);
        }
      }
    }
  hipError_t e = rt_malloc((void**)&p.fzh, out.size() * sizeof(uint16_t));
  if (e == hipSuccess) e = rt_copy_to_device(p.fzh, out.data(), out.size() * sizeof(uint16_t));
  if (e != hipSuccess) return e;
  p.fzh_off2 = per;
  p.fzh_gs = groups > 1 ? kFbBlockHalves : 0;
  p.fzh_n = per;
  p.fzh_exact = exact ? 1 : 0;
  return hipSuccess;
}

}  // namespace

// Stage-0 blocks for the fast path: zero-padded to 16*nb, with the plan's
// signs folded in.  M = ... B_0 D, and the members of stage-0 group c are
// i = k*S_0 + c (S_0 = 256), so (B_0 D) restricted to group c is
// B_{0,c} diag(s[k*256 + c]): column k of the block times that sign.  Each
// entry x is split into hi = f16(x), lo = f16(x - hi) (nearest even), laid out
// for pass A's U_0 (radix 16: fb_hentry) and V_0 (fa_vhentry).  The fast path
// is refused (fz_ok stays 0) when a block row has norm above 1 + 1e-3.
hipError_t fused_prepare(Plan& p, const float* host_blocks, const int8_t* host_signs) {
  const hipError_t es = prepare_split16(p, host_blocks);
  if (es != hipSuccess) return es;
  const int b0 = fused_b0(p);
  if (!b0 || !p.fzh) return hipSuccess;
  const int nb = (b0 + 15) / 16;
  const int np = 16 * nb;
  const int S0 = fused_s0(p);
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
    for (int j = 0; j < b0; ++j) {
      double nrm = 0;
      for (int k = 0; k < b0; ++k) {
        const float sg = host_signs ? (float)host_signs[(size_t)k * S0 + g] : 1.0f;
        const float x = blk[j * b0 + k] * sg;
        pad[((size_t)g * np + j) * np + k] = x;
        nrm += (double)x * x;
      }
      if (!(nrm <= 1.002)) return hipSuccess;  // (1 + 1e-3)^2, and not NaN
    }
  }
  bool exact = true;
  auto split = [&](float x, uint16_t* hi_out, uint16_t* lo_out) {
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);
    if ((float)lo != 0.0f) exact = false;
    *hi_out = __builtin_bit_cast(uint16_t, hi);
    *lo_out = __builtin_bit_cast(uint16_t, lo);
  };
  // V_0 order: entry (nt, lr, lg, ch) holds V[16 nt + lr][16 ch + 4 lg + i]
  const int64_t gv = (int64_t)kFbBlockHalves * nb * nb;
  std::vector<uint16_t> v0((size_t)(ng0 * gv));
  for (int g = 0; g < ng0; ++g)
    for (int nt = 0; nt < nb; ++nt)
      for (int lr = 0; lr < 16; ++lr)
        for (int lg = 0; lg < 4; ++lg)
          for (int ch = 0; ch < nb; ++ch) {
            uint16_t* e = v0.data() + g * gv + fa_vhentry(nb, nt, lr, lg, ch);
            for (int i = 0; i < 4; ++i)
              split(pad[((size_t)g * np + 16 * nt + lr) * np + 16 * ch + 4 * lg + i], e + i, e + 4 + i);
          }
  // U_0 order (radix 16 or 32 only): entry (j, q) holds U[j][4 q + i]
  std::vector<uint16_t> u0;
  const int64_t gu = 2 * (int64_t)b0 * b0;  // halves per U_0 block
  if (b0 == 16 || b0 == 32) {
    u0.resize((size_t)(ng0 * gu));
    for (int g = 0; g < ng0; ++g)
      for (int j = 0; j < b0; ++j)
        for (int k = 0; k < b0; ++k) {
          uint16_t* e = u0.data() + g * gu + fa_uhentry(b0, j, k / 4);
          split(pad[((size_t)g * np + j) * np + k], e + k % 4, e + 4 + k % 4);
        }
  }
  hipError_t e = rt_malloc((void**)&p.fz0v, v0.size() * sizeof(uint16_t));
  if (e == hipSuccess) e = rt_copy_to_device(p.fz0v, v0.data(), v0.size() * sizeof(uint16_t));
  if (e == hipSuccess && !u0.empty()) {
    e = rt_malloc((void**)&p.fz0u, u0.size() * sizeof(uint16_t));
    if (e == hipSuccess) e = rt_copy_to_device(p.fz0u, u0.data(), u0.size() * sizeof(uint16_t));
  }
  if (e != hipSuccess) return e;
  p.fz_b0 = b0;
  p.fz_s0 = S0;
  p.fz_nb = nb;
  p.fz_gs0v = per_group ? gv : 0;
  p.fz_gs0u = per_group ? gu : 0;
  p.fz_n0v = (int64_t)v0.size();
  p.fz_n0u = (int64_t)u0.size();
  p.fz0_exact = exact ? 1 : 0;
  p.fz_ok = 1;
  return hipSuccess;
}

namespace {

// Persistent pass B: at most one workgroup per compute unit (its LDS use
// allows no more), and as few as take the tiles in the same number of rounds
// (688 tiles: 230 workgroups of three tiles, not 256 of which 176 take a
// third), so the rounds run with fewer workgroups competing for memory.
int fused_b_grid(const FusedBArgs& b) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (rt_get_device(&dev) != hipSuccess || rt_cu_count(dev, &cus) != hipSuccess || cus < 1)
      cus = 256;
  }
  const int64_t nt = fb_nwg(b);
  const int64_t rounds = (nt + cus - 1) / cus;
  return (int)((nt + rounds - 1) / rounds);
}

const char* check_b(const FusedBArgs& b);

// Host check of what the two kernels' index arithmetic relies on.
const char* check_fused(const FusedAArgs& a, const FusedBArgs& b) {
  if (a.bv < 2 || a.bv > 64 || a.nb != (a.bv + 15) / 16) return "V_0 radix";
  if ((a.ru != 16 && a.ru != 32) || (a.ru == 32 && a.nb > 2)) return "U_0 radix";
  const int P = fa_p(a.wt, a.nb);
  if ((a.qc != 8 && a.qc != 16 && a.qc != 32) || a.su % a.qc || a.sv % P ||
      (int64_t)a.ru * a.su != a.m || a.dv != a.bv * a.sv ||
      (int64_t)a.nchunk * a.dv != a.n)
    return "shape";
  if (fa_nwg(a) % 8 || a.pt < 1 || (a.sv / fa_p(a.wt, a.nb)) % a.pt) return "pass A grid";
  if (fa_lds_bytes(fa_geom(a.wt, a.nb, a.bv, a.ru)) > 160 * 1024) return "pass A LDS";
  // pass A addresses a lane's input and output as 32-bit byte offsets from a
  // per-chunk base
  if ((int64_t)a.m * a.ldw * fa_esz(a.wt) >= (int64_t(1) << 31) ||
      (int64_t)a.m * a.n * 4 >= (int64_t(1) << 31))
    return "32-bit offsets";
  if (!a.w || !a.ws || !a.u0 || !a.v0) return "pass A pointers";
  const int64_t gu = 2 * (int64_t)a.ru * a.ru;
  if (a.u0_n < (a.u0_gs ? a.su * a.u0_gs : gu)) return "U_0 extent";
  if (a.v0_n < (a.v0_gs ? a.sv * a.v0_gs : (int64_t)kFbBlockHalves * a.nb * a.nb)) return "V_0 extent";
  if ((a.u0_gs && a.u0_gs < gu) || (a.v0_gs && a.v0_gs < (int64_t)kFbBlockHalves * a.nb * a.nb) ||
      a.u0_gs % 8 || a.v0_gs % 8)
    return "block strides";
  if (b.m != a.m || b.n != a.n) return "pass B shape";
  return check_b(b);
}

// Host check of pass B alone.
const char* check_b(const FusedBArgs& b) {
  if (b.m < 256 || b.m % 256 || b.nrb != b.m / 256 || b.dv != b.bv * 256 || b.bv < 1 ||
      (int64_t)b.nchunk * b.dv != b.n)
    return "pass B shape";
  if ((int64_t)b.m * b.n * 4 >= (int64_t(1) << 40)) return "pass B extent";
  if (!b.ws || !b.u1 || !b.u2 || !b.v1 || !b.v2 || !b.codes || !b.scales) return "pass B pointers";
  if (b.u1_n < (b.u1_gs ? (int64_t)b.nrb * 16 * b.u1_gs : kFbBlockHalves)) return "U_1 extent";
  if (b.u2_n < (b.u2_gs ? (int64_t)b.nrb * 16 * b.u2_gs : kFbBlockHalves)) return "U_2 extent";
  if (b.v1_n < (b.v1_gs ? (int64_t)b.bv * 16 * b.v1_gs : kFbBlockHalves)) return "V_1 extent";
  if (b.v2_n < (b.v2_gs ? (int64_t)b.bv * 16 * b.v2_gs : kFbBlockHalves)) return "V_2 extent";
  if ((b.u1_gs && b.u1_gs < kFbBlockHalves) || (b.v1_gs && b.v1_gs < kFbBlockHalves) ||
      b.u1_gs % 8 || b.v1_gs % 8 || b.u2_gs != b.u1_gs || b.v2_gs != b.v1_gs)
    return "block strides";
  if (b.group != 64 && b.group != 128) return "group";
  if (b.bits < 2 || b.bits > 5 || b.nlev != (1 << b.bits)) return "bits";
  if (b.codes_ld * 8 != b.n * b.bits || b.codes_ld % 4 || b.scales_ld * b.group != b.n)
    return "code layout";
  return nullptr;
}

// Pass B's split blocks of both sides.
void set_split_blocks(FusedBArgs& b, const Plan* U, const Plan* V) {
  b.u1 = U->fzh;
  b.u2 = U->fzh + U->fzh_off2;
  b.u1_gs = b.u2_gs = U->fzh_gs;
  b.u1_n = b.u2_n = U->fzh_n;
  b.v1 = V->fzh;
  b.v2 = V->fzh + V->fzh_off2;
  b.v1_gs = b.v2_gs = V->fzh_gs;
  b.v1_n = b.v2_n = V->fzh_n;
  b.exact = U->fzh_exact && V->fzh_exact ? 1 : 0;
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
  rt_free(p.fz0u);
  rt_free(p.fz0v);
  rt_free(p.fzh);
  p.fz0u = p.fz0v = nullptr;
  p.fzh = nullptr;
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
  if (!U || !V || !U->fz_ok || !V->fz_ok || !U->fzh || !V->fzh) return false;
  if ((U->fz_b0 != 16 && U->fz_b0 != 32) || U->d != m || n % V->d) return false;
  if (U->fz_b0 == 32 && V->fz_nb > 2) return false;
  if (q->group != 64 && q->group != 128) return false;
  if ((n * q->bits) % 32) return false;
  const int elem = wt == BRQ_F32 ? 4 : 2;
  if ((ldw * elem) % 16 || reinterpret_cast<uintptr_t>(w) % 16) return false;
  // stages between stage 0 and the last two run as stage passes in place
  if ((mid_stages(*U) && !sp_shape_ok(U, 1, m, n)) || (mid_stages(*V) && !sp_shape_ok(V, 0, m, n)))
    return false;
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
  a.ru = U->fz_b0;
  a.su = U->fz_s0;
  a.sv = V->fz_s0;
  a.dv = V->d;
  a.nchunk = (int)(n / V->d);
  a.u0 = U->fz0u;
  a.u0_gs = U->fz_gs0u;
  a.u0_exact = U->fz0_exact;
  a.v0 = V->fz0v;
  a.v0_gs = V->fz_gs0v;
  {
    int dev = 0, cus = 0;
    if (rt_get_device(&dev) != hipSuccess || rt_cu_count(dev, &cus) != hipSuccess || cus < 1) return BRQ_ERR_HIP;
    a.qc = kFaQC;
    a.qc = fa_qc(a.su % kFaQC ? 0 : fa_nwg(a), a.su, cus);
    a.pt = a.su % a.qc ? 1 : fa_pt(a, fa_nwg(a), cus);
  }

  FusedBArgs b;
  std::memset(&b, 0, sizeof b);
  b.ws = a.ws;
  b.m = m;
  b.n = n;
  b.nrb = (int)(m / 256);
  b.bv = V->d / 256;
  b.nchunk = a.nchunk;
  b.dv = a.dv;
  set_split_blocks(b, U, V);
  fill_quant_b(b, q, n);
  b.codes = codes;
  b.scales = scales;
  a.u0_n = U->fz_n0u;
  a.v0_n = V->fz_n0v;
  if (check_fused(a, b)) return BRQ_ERR_UNSUPPORTED;

  char name[96];
  snprintf(name, sizeof name, "fusedA U0(%d) V0(%d)", a.ru, a.bv);
  int tok = prof_begin(name, s);
  hipError_t e = launch_fused_a(a, s);
  prof_end(tok, s);
  if (e != hipSuccess) return BRQ_ERR_HIP;
  // the stages between stage 0 and the last two, in place on the intermediate
  for (int side = 1; side >= 0; --side) {
    const Plan* p = side ? U : V;
    if (!mid_stages(*p)) continue;
    hipError_t he = hipSuccess;
    const brq_status st = sp_rotate_stages(p, side, 0, 1, p->nst - 2, ws, BRQ_F32, n, ws, BRQ_F32, n, m, n,
                                           nullptr, 0, s, &he);
    if (st != BRQ_OK) return st == BRQ_ERR_HIP ? BRQ_ERR_HIP : BRQ_ERR_UNSUPPORTED;
  }
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
  if (!dense_tail16(U) || !dense_tail16(V) || !U->fzh || !V->fzh || U->d != m || n % V->d) return false;
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
  set_split_blocks(b, U, V);
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
