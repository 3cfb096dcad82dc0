// Host dry run of libbrq: plans live in host memory and every kernel launch is
// replaced by a walk over each index the kernel would touch, checked against
// the extents of its buffers.  Built as libbrq_dryrun.so for CPU tests; it
// never touches a GPU.  Device pointers passed to it are never dereferenced.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "brq_internal.h"
#include "harp.h"
#include "orp.h"
#include "qlinear.h"

namespace brq {

static std::string g_violation;
static long long g_launches = 0;
static long long g_rows_launches = 0;  // of those, left-side stages by whole rows
static long long g_lanes_launches = 0;  // right-side stages with groups in lanes
static long long g_harp_batches = 0;    // batched HARP block launches
static long long g_pair2_launches = 0;  // two-stage pair launches

static bool violation(const char* fmt, long long a, long long b) {
  if (g_violation.empty()) {
    char buf[256];
    snprintf(buf, sizeof buf, fmt, a, b);
    g_violation = buf;
    fprintf(stderr, "[dryrun] %s\n", buf);
  }
  return false;
}

hipError_t rt_get_device(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t rt_malloc(void** p, size_t bytes) {
  *p = std::malloc(bytes ? bytes : 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t rt_copy_to_device(void* dst, const void* src, size_t bytes) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t rt_copy_to_host(void* dst, const void* src, size_t bytes) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t rt_cu_count(int, int* cus) {
  *cus = 256;
  return hipSuccess;
}

void rt_free(void* p) { std::free(p); }

// Number of float elements of the block array one stage may address.
static int64_t stage_block_floats(const StageDesc& st, const AxisDesc& ax) {
  if (st.mode == BRQ_PER_GROUP) return (int64_t)(ax.d / st.b) * st.b * st.b;
  if (st.mode == BRQ_SHARED) return (int64_t)st.b * st.b;
  return 0;
}

static bool walk_stage(const StageDesc& st, const AxisDesc& ax, int axis, int64_t relbase,
                       int nlines, int ldl, int64_t lds_floats) {
  const int ngroups = (ax.P / st.b) * ax.W;
  std::vector<int> touched((size_t)ax.P * ax.W, 0);
  for (int gid = 0; gid < ngroups; ++gid) {
    const TileGroup tg = tile_group(st, ax, gid);
    for (int j = 0; j < st.b; ++j) {
      const int e = tg.e0 + j * tg.estep;
      if (e < 0 || e >= ax.P * ax.W) return violation("stage member %lld outside the tile (%lld)", e, ax.P * ax.W);
      touched[e]++;
      for (int line : {0, nlines - 1}) {
        const int64_t a = axis ? (int64_t)line * ldl + e : (int64_t)e * ldl + line;
        if (a < 0 || a >= lds_floats) return violation("LDS index %lld >= %lld", a, lds_floats);
      }
    }
    if (st.mode == BRQ_PER_GROUP) {
      const int64_t c = group_index(st, ax, relbase, tg);
      const int64_t hi = (c + 1) * st.b * st.b;
      if (c < 0 || hi > stage_block_floats(st, ax)) return violation("block group %lld of %lld", c, ax.d / st.b);
    }
  }
  for (size_t e = 0; e < touched.size(); ++e)
    if (touched[e] != 1) return violation("tile element %lld updated %lld times", (long long)e, touched[e]);
  return true;
}

hipError_t launch_pass(const PassArgs& a, hipStream_t) {
  ++g_launches;
  const AxisDesc& X0 = a.ax[0];
  const AxisDesc& X1 = a.ax[1];
  const int64_t tr = axis_tiles(X0), tc = axis_tiles(X1);
  const int RT = X0.P * X0.W, CT = X1.P * X1.W, ldl = CT + 1;
  const int64_t lds_floats = (int64_t)RT * ldl;
  std::vector<uint8_t> cover((size_t)(a.m * a.n), 0);
  for (int64_t t = 0; t < tr * tc; ++t) {
    const int64_t ir = t / tc, ic = t - (t / tc) * tc;
    const AxisPos pr = axis_pos(X0, ir), pc = axis_pos(X1, ic);
    for (int er = 0; er < RT; ++er) {
      if (er >= pr.limit) continue;
      const int64_t row = pr.base + axis_off(X0, er);
      if (row < 0 || row >= a.m) return violation("row %lld outside [0, %lld)", row, a.m), hipErrorInvalidValue;
      for (int ec = 0; ec < CT; ++ec) {
        if (ec >= pc.limit) continue;
        const int64_t col = pc.base + axis_off(X1, ec);
        if (col < 0 || col >= a.n) return violation("col %lld outside [0, %lld)", col, a.n), hipErrorInvalidValue;
        if (a.pro == PRO_LOAD && col >= a.ld_src) return violation("col %lld >= ld_src %lld", col, a.ld_src), hipErrorInvalidValue;
        if (a.epi == EPI_STORE && col >= a.ld_dst) return violation("col %lld >= ld_dst %lld", col, a.ld_dst), hipErrorInvalidValue;
        if (a.pro == PRO_DEQUANT && (col * a.bits) / 8 >= a.codes_ld)
          return violation("code byte %lld >= %lld", (col * a.bits) / 8, a.codes_ld), hipErrorInvalidValue;
        if (X1.sign && X1.sign_mod < 1) return violation("sign length %lld %lld", X1.sign_mod, 0), hipErrorInvalidValue;
        cover[(size_t)(row * a.n + col)]++;
      }
    }
    for (int s = 0; s < X0.nst; ++s)
      if (!walk_stage(X0.st[s], X0, 0, pr.relbase, CT, ldl, lds_floats)) return hipErrorInvalidValue;
    for (int s = 0; s < X1.nst; ++s)
      if (!walk_stage(X1.st[s], X1, 1, pc.relbase, RT, ldl, lds_floats)) return hipErrorInvalidValue;
    if (a.epi == EPI_QUANT) {
      const int g = a.group, gpr = CT / g, nbytes = g * a.bits / 8;
      if (g > 1024) return violation("group %lld > %lld", g, 1024), hipErrorInvalidValue;
      for (int u = 0; u < RT * gpr; ++u) {
        const int er = u / gpr, gi = u % gpr;
        if (er >= pr.limit || (int64_t)gi * g >= pc.limit) continue;
        const int64_t row = pr.base + er;
        if ((pc.base + (int64_t)gi * g) % g) return violation("group start %lld not aligned to %lld", pc.base + gi * g, g), hipErrorInvalidValue;
        const int64_t gcol = (pc.base + (int64_t)gi * g) / g;
        const int64_t off = row * a.codes_ld + gcol * nbytes;
        if (off < 0 || off + nbytes > a.m * a.codes_ld) return violation("codes [%lld, +%lld) outside", off, nbytes), hipErrorInvalidValue;
        if (row * a.scales_ld + gcol >= a.m * a.scales_ld) return violation("scale %lld of %lld", row * a.scales_ld + gcol, a.m * a.scales_ld), hipErrorInvalidValue;
        if ((int64_t)er * ldl + (int64_t)gi * g + g > lds_floats) return violation("quant LDS %lld > %lld", (int64_t)er * ldl + gi * g + g, lds_floats), hipErrorInvalidValue;
      }
    }
  }
  for (int64_t i = 0; i < a.m * a.n; ++i)
    if (cover[(size_t)i] != 1) return violation("element %lld covered %lld times", i, cover[(size_t)i]), hipErrorInvalidValue;
  return hipSuccess;
}

}  // namespace brq

extern "C" {
// Dry-run diagnostics (only in libbrq_dryrun.so).
const char* brq_dryrun_violation(void) { return brq::g_violation.c_str(); }
long long brq_dryrun_launches(void) { return brq::g_launches; }
long long brq_dryrun_rows_launches(void) { return brq::g_rows_launches; }
long long brq_dryrun_harp_batches(void) { return brq::g_harp_batches; }
long long brq_dryrun_pair2_launches(void) { return brq::g_pair2_launches; }
long long brq_dryrun_lanes_launches(void) { return brq::g_lanes_launches; }
void brq_dryrun_reset(void) {
  brq::g_violation.clear();
  brq::g_launches = 0;
  brq::g_rows_launches = 0;
  brq::g_lanes_launches = 0;
  brq::g_harp_batches = 0;
  brq::g_pair2_launches = 0;
}
}

// Kernel timing is meaningless without a device: the calls exist and report
// no kernels.
namespace brq {
int prof_begin(const char*, hipStream_t) { return -1; }
void prof_end(int, hipStream_t) {}
}  // namespace brq

extern "C" {
brq_status brq_profile_enable(int32_t) { return BRQ_OK; }
brq_status brq_profile_reset(void) { return BRQ_OK; }
int32_t brq_profile_count(void) { return 0; }
brq_status brq_profile_read(int32_t, char*, size_t, double*, int64_t*) {
  return BRQ_ERR_INVALID_ARGUMENT;
}
}

// ---------------------------------------------------------------- fast path

#include "fused.h"

namespace brq {

static bool in_range(int64_t lo, int64_t n, int64_t extent) { return lo >= 0 && lo + n <= extent; }

hipError_t launch_fused_a(const FusedAArgs& a, hipStream_t) {
  ++g_launches;
  const int64_t nwg = fa_nwg(a);
  const int nb = a.nb, bv = a.bv, ru = a.ru;
  if (ru != 16 && ru != 32) return violation("pass A U_0 radix %lld", ru, 0), hipErrorInvalidValue;
  const FaGeom g = fa_geom(a.wt, nb, bv, ru);
  const int st = fa_steps(bv), ki = fa_ki(a.wt, st, ru), kq = fa_kq_nt(a.wt, st, ru);
  const int P = g.P, ppw = g.ppw, esz = g.esz, epi = 16 / esz, ipr = g.ipr;
  if (64 % ipr || a.sv % P || (a.qc != 8 && a.qc != 16 && a.qc != 32) || a.su % a.qc || 8 * ki < ru * fa_ncb(64 / ipr, st) ||
      8 * kq * (64 / (P / 4)) < ru * 16)
    return violation("pass A loop counts %lld / %lld", ki, kq), hipErrorInvalidValue;
  if (fa_lds_bytes(g) > 160 * 1024 || g.slab_bytes % 16 || g.max_off < g.slab_bytes + g.out_floats * 4 ||
      g.max_off % 4 || fa_lds_bytes(g) < g.max_off + 4 * kFaWaves)
    return violation("pass A LDS %lld bytes", fa_lds_bytes(g), 0), hipErrorInvalidValue;
  for (int e = 0; e < 255; ++e) {  // the slab scale puts every maximum in [2^11, 2^12)
    const float mlo = e ? std::ldexp(1.0f, e - 127) : 0.0f;
    uint32_t bits;
    std::memcpy(&bits, &mlo, 4);
    const int ks = fa_scale_shift(bits);
    if (ks != fa_scale_shift(bits | 0x7fffffu)) return violation("slab scale of exponent %lld", e, ks), hipErrorInvalidValue;
    if (e > 0 && std::ldexp((double)mlo, ks) != 2048.0) return violation("slab scale of exponent %lld", e, ks), hipErrorInvalidValue;
    if (e == 0 && std::ldexp(std::ldexp(1.0, -126), ks) > 4096.0) return violation("slab scale of subnormals", 0, ks), hipErrorInvalidValue;
  }
  // which input element (r0, c0, p_local) each slab byte holds, and which
  // output (r0', c0', p_local) each float of the output area holds
  auto code = [&](int r0, int c0, int pl) { return ((int64_t)r0 * 64 + c0) * 256 + pl; };
  std::vector<int64_t> slab(g.slab_bytes), outa(g.out_floats);
  std::vector<uint8_t> cover((size_t)(a.m * a.n), 0);
  for (int64_t b = 0; b < nwg; ++b) {
    const FaTile t = fa_tile(a, b, nwg);
    if (t.p0 < 0 || t.p0 + P > a.sv || t.p0 % P || t.q0 < 0 || t.q0 + a.qc > a.su || t.chunk < 0 ||
        t.chunk >= a.nchunk)
      return violation("pass A tile %lld of %lld", b, nwg), hipErrorInvalidValue;
    for (int w = 0; w < kFaWaves; ++w)
      for (int j = 0; j < ppw; ++j)
        for (int l = 0; l < 64; ++l)
          for (int nt = 0; nt < nb; ++nt)
            for (int ch = 0; ch < nb; ++ch) {
              const int64_t i = (int64_t)(t.p0 + ppw * w + j) * a.v0_gs + fa_vhentry(nb, nt, l & 15, l >> 4, ch);
              if (!in_range(i, 8, a.v0_n) || i % 8)
                return violation("V_0 block read (p %lld, lane %lld)", t.p0 + ppw * w + j, l), hipErrorInvalidValue;
            }
    for (int q = t.q0; q < t.q0 + a.qc; ++q) {
      std::fill(slab.begin(), slab.end(), -1);
      std::fill(outa.begin(), outa.end(), -1);
      std::vector<uint8_t> loaded(g.items, 0);
      for (int w = 0; w < kFaWaves; ++w)
        for (int l = 0; l < 64; ++l) {
          const int o = l % ipr;
          for (int k = 0; k < ki; ++k) {
            const FaSlot x = fa_slot(ipr, w, k, l, bv, 0, ru);
            const int r0 = x.r0, c0 = x.c0;
            if (c0 < 0 || c0 >= bv || r0 >= ru) return violation("pass A load column %lld", c0, 0), hipErrorInvalidValue;
            loaded[(size_t)((r0 * bv + c0) * ipr + o)] = 1;
            const int64_t row = fa_row(a, r0, q), col = fa_col(a, t.chunk, c0, t.p0 + o * epi);
            if (row >= a.m || !in_range(col, epi, a.n) || col + epi > a.ldw || ((row * a.ldw + col) * esz) % 16)
              return violation("pass A input (%lld, %lld)", row, col), hipErrorInvalidValue;
            // the kernel's 32-bit lane offset: (r0 * su * ldw + c0 * sv + o * epi) * esz
            if (((int64_t)r0 * a.su * a.ldw + (int64_t)c0 * a.sv + o * epi) * esz >= (int64_t(1) << 32))
              return violation("pass A 32-bit input offset (%lld, %lld)", r0, c0), hipErrorInvalidValue;
            const int off = fa_slab_item(g, r0, c0, o);
            if (!in_range(off, 16, g.slab_bytes) || off % 8)
              return violation("pass A slab write at byte %lld", off, 0), hipErrorInvalidValue;
            for (int e = 0; e < epi; ++e) {
              const int64_t c = code(r0, c0, o * epi + e);
              for (int bb = 0; bb < esz; ++bb) {
                int64_t& sl = slab[(size_t)(off + e * esz + bb)];
                if (sl != -1 && sl != c) return violation("pass A slab byte %lld written twice", off + e * esz + bb, 0), hipErrorInvalidValue;
                sl = c;
              }
            }
          }
        }
      for (int it = 0; it < g.items; ++it)
        if (!loaded[it]) return violation("pass A item %lld not loaded", it, 0), hipErrorInvalidValue;
      for (int w = 0; w < kFaWaves; ++w)
        for (int l = 0; l < 64; ++l) {
          const int lr = l & 15, lg = l >> 4;
          for (int ot = 0; ot < ru / 16; ++ot)
            for (int kt = 0; kt < ru / 16; ++kt)
              if (!in_range((int64_t)q * a.u0_gs + fa_uhentry(ru, 16 * ot + lr, 4 * kt + lg), 8, a.u0_n))
                return violation("U_0 block read q %lld lane %lld", q, l), hipErrorInvalidValue;
          for (int mt = 0; mt < ru / 16; ++mt)
            for (int ci = 0; ci < 16 * nb; ++ci) {  // chunk ci / 16, (ci / 4) % 4 == lg, i = ci % 4
              if (((ci / 4) & 3) != lg) continue;
              const int c0 = std::min(ci, bv - 1);
              const int off = fa_slab_read(g, 16 * mt + lr, c0, w);
              if (!in_range(off, ppw * esz, g.slab_bytes) || off % (ppw * esz))
                return violation("pass A slab read at byte %lld", off, 0), hipErrorInvalidValue;
              for (int e = 0; e < ppw; ++e)
                for (int bb = 0; bb < esz; ++bb)
                  if (slab[(size_t)(off + e * esz + bb)] != code(16 * mt + lr, c0, ppw * w + e))
                    return violation("pass A slab read of the wrong element at byte %lld", off + e * esz + bb, 0), hipErrorInvalidValue;
            }
          for (int nt = 0; nt < nb; ++nt)
            for (int ot = 0; ot < ru / 16; ++ot)
              for (int i = 0; i < 4; ++i) {
                const int c0 = 16 * nt + 4 * lg + i;
                if (c0 >= bv) continue;
                const int off = fa_out(g, 16 * ot + lr, c0, ppw * w);
                if (!in_range(off, ppw, g.out_floats) || (off * 4) % (ppw * 4))
                  return violation("pass A output-area write %lld", off, 0), hipErrorInvalidValue;
                for (int e = 0; e < ppw; ++e) {
                  int64_t& s = outa[(size_t)(off + e)];
                  if (s != -1) return violation("pass A output float %lld written twice", off + e, 0), hipErrorInvalidValue;
                  s = code(16 * ot + lr, c0, ppw * w + e);
                }
              }
        }
      std::vector<uint8_t> stored((size_t)ru * bv * (P / 4), 0);
      for (int w = 0; w < kFaWaves; ++w)
        for (int l = 0; l < 64; ++l) {
          const int pq = l % (P / 4);
          for (int k = 0; k < kq * nb; ++k) {
            const int nt = k / kq;
            const FaSlot x = fa_slot(P / 4, w, k % kq, l, bv, 16 * nt, ru);
            const int r0 = x.r0, c0 = x.c0;
            if (c0 < 16 * nt || c0 >= 16 * nt + 16)
              return violation("pass A store column %lld outside tile %lld", c0, nt), hipErrorInvalidValue;
            {
              if (r0 >= ru || c0 < 0 || c0 >= bv) return violation("pass A store row %lld col %lld", r0, c0), hipErrorInvalidValue;
              const int off = fa_out(g, r0, c0, 4 * pq);
              if (!in_range(off, 4, g.out_floats) || off % 4)
                return violation("pass A output-area read %lld", off, 0), hipErrorInvalidValue;
              for (int e = 0; e < 4; ++e)
                if (outa[(size_t)(off + e)] != code(r0, c0, 4 * pq + e))
                  return violation("pass A output-area read of the wrong value at %lld", off + e, 0), hipErrorInvalidValue;
              const int64_t row = fa_row(a, r0, q), col = fa_col(a, t.chunk, c0, t.p0 + 4 * pq);
              if (row >= a.m || !in_range(col, 4, a.n) || (row * a.n + col) % 4)
                return violation("pass A store (%lld, %lld)", row, col), hipErrorInvalidValue;
              if (((int64_t)r0 * a.su * a.n + (int64_t)c0 * a.sv + 4 * pq) * 4 >= (int64_t(1) << 32))
                return violation("pass A 32-bit output offset (%lld, %lld)", r0, c0), hipErrorInvalidValue;
              uint8_t& sd = stored[(size_t)((r0 * bv + c0) * (P / 4) + pq)];
              if (!sd)  // a repeated last column stores the same value again
                for (int e = 0; e < 4; ++e) cover[(size_t)(row * a.n + col + e)]++;
              sd = 1;
            }
          }
        }
      for (size_t i = 0; i < stored.size(); ++i)
        if (!stored[i]) return violation("pass A output float4 %lld not stored", (int64_t)i, 0), hipErrorInvalidValue;
    }
  }
  for (int64_t i = 0; i < a.m * a.n; ++i)
    if (cover[(size_t)i] != 1) return violation("pass A element %lld written %lld times", i, cover[(size_t)i]), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_fused_b(const FusedBArgs& a, int grid, hipStream_t) {
  ++g_launches;
  const int64_t ntiles = fb_nwg(a);
  if (grid < 1 || grid > ntiles) return violation("pass B grid %lld of %lld tiles", grid, ntiles), hipErrorInvalidValue;
  std::vector<uint8_t> cover((size_t)(a.m * a.n), 0);
  std::vector<int> slot(kFbXchFloats), qread(kFbXchFloats);
  const int bits = a.bits, g = a.group;
  std::vector<uint8_t> code_bytes((size_t)(a.m * a.codes_ld), 0), scale_seen((size_t)(a.m * a.scales_ld), 0);
  std::vector<int> tiles_seen((size_t)ntiles, 0);
  for (int e = 0; e < 255; ++e) {  // the tile scale puts every maximum in [64, 128), or scales by 2^127
    const float mlo = e ? std::ldexp(1.0f, e - 127) : 0.0f;
    uint32_t bits;
    std::memcpy(&bits, &mlo, 4);
    const int ks = fb_scale_shift(bits), ks2 = fb_scale_shift(bits | 0x7fffffu);
    if (ks != ks2 || ks > 127 || ks < -126) return violation("tile scale of exponent %lld: %lld", e, ks), hipErrorInvalidValue;
    if (e >= 6 && (std::ldexp((double)mlo, ks) != 64.0)) return violation("tile scale of exponent %lld", e, ks), hipErrorInvalidValue;
    if (e < 6 && ks != 127) return violation("tile scale of small exponent %lld", e, ks), hipErrorInvalidValue;
  }
  {  // the V_1 row order is a permutation of the 16 rows
    int seen = 0;
    for (int n = 0; n < 16; ++n) seen |= 1 << fb_sigma(n);
    if (seen != 0xffff) return violation("V_1 row order is not a permutation", 0, 0), hipErrorInvalidValue;
  }
  for (int64_t wg = 0; wg < grid; ++wg)
    for (int64_t tile = wg; tile < ntiles; tile += grid) {  // the kernel's persistent loop
      tiles_seen[(size_t)tile]++;
      const FbTile t = fb_tile(a, tile);
      if (t.r0 < 0 || t.r0 >= a.nrb || a.nrb * 256 != a.m || t.c0 < 0 || t.c0 >= a.bv || t.chunk < 0 ||
          t.chunk >= a.nchunk)
        return violation("pass B tile %lld of %lld", tile, ntiles), hipErrorInvalidValue;
      {  // each staged block's quads are a permutation of its 64 slots
        std::vector<int> seen(256, 0);
        for (int qd = 0; qd < 64; ++qd) {
          const int o = fb_vslot(qd >> 2, qd & 3);
          if (o < 0 || o + 4 > 256 || o % 4) return violation("V block slot %lld of quad %lld", o, qd), hipErrorInvalidValue;
          for (int j = 0; j < 4; ++j) seen[o + j]++;
        }
        for (int i = 0; i < 256; ++i)
          if (seen[i] != 1) return violation("V block float %lld staged %lld times", i, seen[i]), hipErrorInvalidValue;
      }
      // block staging into LDS: (bh, bh) entries, and (bl, bl) unless exact;
      // the maxima between the V_1 blocks and the end of the exchange buffer
      if (kFbV1LOff + 16 * 256 > kFbMaxOff || kFbMaxOff + 16 > kFbXchFloats || kFbV2Off != kFbXchFloats ||
          kFbV2LOff != kFbV2Off + 16 * 256 || kFbLdsFloats != kFbV2LOff + 16 * 256 ||
          kFbLdsFloats * 4 > 160 * 1024)
        return violation("pass B LDS layout", 0, 0), hipErrorInvalidValue;
      for (int k = 0; k < 2 * 16 * 64; ++k) {
        const int which = k >> 10, rem = k & 1023, f = rem >> 6, qd = rem & 63;
        const int64_t src = (int64_t)(t.c0 * 16 + f) * (which ? a.v2_gs : a.v1_gs) + fb_hentry(qd >> 2, qd & 3);
        if (!in_range(src, 8, which ? a.v2_n : a.v1_n) || src % 8)
          return violation("V block staging %lld", src, which), hipErrorInvalidValue;
        const int dst = (which ? kFbV2Off : kFbV1Off) + f * 256 + fb_vslot(qd >> 2, qd & 3);
        if (!in_range(dst, 4, kFbLdsFloats) || (which == 0 && dst + 4 > kFbV1LOff) ||
            (which == 1 && dst + 4 > kFbV2LOff) || dst % 4)
          return violation("V block LDS slot %lld", dst, which), hipErrorInvalidValue;
        const int dl = (which ? kFbV2LOff : kFbV1LOff) + f * 256 + fb_vslot(qd >> 2, qd & 3);
        if (!in_range(dl, 4, kFbLdsFloats) || (which == 0 && dl + 4 > kFbMaxOff) || dl % 4)
          return violation("V bl LDS slot %lld", dl, which), hipErrorInvalidValue;
      }
      for (int w = 0; w < kFbWaves; ++w)
        for (int l = 0; l < 64; ++l) {
          const int lr = l & 15, lg = l >> 4;
          // the two halves fb_load_half<H>: columns c1 = 4 lg + 2H + e, all c2
          const int64_t row = fb_row(t, lr, w);
          for (int hh = 0; hh < 2; ++hh)
            for (int e = 0; e < 2; ++e)
              for (int qd = 0; qd < 4; ++qd) {
                const int64_t col = fb_col(a, t, 4 * lg + 2 * hh, 0) + e * 16 + 4 * qd;
                const int64_t off = row * a.n + col;
                if (row >= a.m || !in_range(col, 4, a.n) || off % 4)
                  return violation("pass B load (%lld, %lld)", row, col), hipErrorInvalidValue;
                for (int j = 0; j < 4; ++j) cover[(size_t)(off + j)]++;
              }
          if (!in_range((int64_t)(t.r0 * 16 + w) * a.u1_gs + fb_hentry(lr, lg), 8, a.u1_n) ||
              !in_range((int64_t)(t.r0 * 16 + w) * a.u2_gs + fb_hentry(lr, lg), 8, a.u2_n))
            return violation("U_1/U_2 block read wave %lld lane %lld", w, l), hipErrorInvalidValue;
          for (int c = 0; c < 16; ++c) {
            if (!in_range(kFbV1Off + c * 256 + fb_vslot(fb_sigma(lr), lg), 4, kFbV1LOff) ||
                !in_range(kFbV2Off + c * 256 + fb_vslot(lr, lg), 4, kFbV2LOff) ||
                !in_range(kFbV1LOff + c * 256 + fb_vslot(fb_sigma(lr), lg), 4, kFbMaxOff) ||
                !in_range(kFbV2LOff + c * 256 + fb_vslot(lr, lg), 4, kFbLdsFloats))
              return violation("V block LDS read %lld lane %lld", c, l), hipErrorInvalidValue;
          }
        }
      for (int h = 0; h < 2; ++h) {
        std::fill(slot.begin(), slot.end(), 0);
        std::fill(qread.begin(), qread.end(), 0);
        for (int w = 0; w < kFbWaves; ++w)
          for (int l = 0; l < 64; ++l) {
            const int lr = l & 15, lg = l >> 4;
            // registers j = 2h + e hold c1' = lg + 4 j, i.e. c1h = lg + 4 e
            for (int e = 0; e < 2; ++e)
              for (int qd = 0; qd < 4; ++qd) {
                const int c1h = lg + 4 * e;
                if (fb_sigma(4 * lg + 2 * h + e) != 8 * h + c1h)
                  return violation("phase-1 output order %lld %lld", lg, e), hipErrorInvalidValue;
                const int s = fb_xch(lr, c1h, w, 4 * qd);
                if (!in_range(s, 4, kFbXchFloats) || s % 4) return violation("exchange write %lld", s, 0), hipErrorInvalidValue;
                for (int j = 0; j < 4; ++j) {
                  if (fb_xch(lr, c1h, w, 4 * qd + j) != s + j) return violation("exchange write quad %lld", s, j), hipErrorInvalidValue;
                  slot[s + j]++;
                }
              }
          }
        for (int s = 0; s < kFbXchFloats; ++s)
          if (slot[s] != 1) return violation("exchange slot %lld written %lld times", s, slot[s]), hipErrorInvalidValue;
        for (int w = 0; w < kFbWaves; ++w)
          for (int l = 0; l < 64; ++l) {
            const int lr = l & 15, lg = l >> 4;
            for (int c1h = 0; c1h < 8; ++c1h) {
              const int s = fb_xch(w, c1h, lr, 4 * lg);
              if (!in_range(s, 4, kFbXchFloats) || s % 4) return violation("exchange read %lld", s, 0), hipErrorInvalidValue;
              for (int i = 0; i < 4; ++i)
                if (fb_xch(w, c1h, lr, 4 * lg + i) != s + i) return violation("exchange quad %lld", s, i), hipErrorInvalidValue;
            }
            // the quantizer: lane (lr, lg) reads row r2 = lr, c1h = 2 lg + e, all c2
            for (int e = 0; e < 2; ++e)
              for (int q = 0; q < 4; ++q) {
                const int sq = fb_xch(w, 2 * lg + e, lr, 4 * q);
                if (!in_range(sq, 4, kFbXchFloats) || sq % 4)
                  return violation("quantizer read %lld", sq, 0), hipErrorInvalidValue;
                for (int i = 0; i < 4; ++i) {
                  if (fb_xch(w, 2 * lg + e, lr, 4 * q + i) != sq + i)
                    return violation("quantizer quad %lld", sq, i), hipErrorInvalidValue;
                  qread[sq + i]++;
                }
              }
            const int64_t row = fb_row(t, w, lr);
            const int64_t col0 = fb_col(a, t, 8 * h + 2 * lg, 0);
            if (col0 % 32) return violation("quantizer columns start %lld", col0, 0), hipErrorInvalidValue;
            const int64_t off = row * a.codes_ld + col0 * bits / 8;
            if (!in_range(off, 4 * bits, a.m * a.codes_ld) || off % 4)
              return violation("codes [%lld, +%lld)", off, 4 * bits), hipErrorInvalidValue;
            for (int64_t b = off; b < off + 4 * bits; ++b) code_bytes[(size_t)b]++;
            if (fb_scale_lane(lg, g)) {
              const int64_t si = row * a.scales_ld + col0 / g;
              if (!in_range(si, 1, a.m * a.scales_ld))
                return violation("scale %lld", si, 0), hipErrorInvalidValue;
              scale_seen[(size_t)si]++;
            }
          }
        for (int sq = 0; sq < kFbXchFloats; ++sq)  // each half's slots are read exactly once
          if (qread[sq] != 1) return violation("quantizer read slot %lld %lld times", sq, qread[sq]), hipErrorInvalidValue;
      }
    }
  for (size_t b = 0; b < code_bytes.size(); ++b)
    if (code_bytes[b] != 1) return violation("code byte %lld written %lld times", (int64_t)b, code_bytes[b]), hipErrorInvalidValue;
  for (size_t i = 0; i < scale_seen.size(); ++i)
    if (scale_seen[i] != 1) return violation("scale %lld written %lld times", (int64_t)i, scale_seen[i]), hipErrorInvalidValue;
  for (int64_t i = 0; i < ntiles; ++i)
    if (tiles_seen[(size_t)i] != 1) return violation("pass B tile %lld visited %lld times", i, tiles_seen[(size_t)i]), hipErrorInvalidValue;
  for (int64_t i = 0; i < a.m * a.n; ++i)
    if (cover[(size_t)i] != 1) return violation("pass B element %lld read %lld times", i, cover[(size_t)i]), hipErrorInvalidValue;
  return hipSuccess;
}

}  // namespace brq

// ---------------------------------------------------------------- row Hadamard

#include "rowhad.h"

namespace brq {

hipError_t launch_rowhad(const RhArgs& a, hipStream_t) {
  ++g_launches;
  const int l2d = a.log2d, d = 1 << l2d, R = rh_rounds(l2d);
  if (a.nchunks > kRhMaxChunks) return violation("row Hadamard chunk count %lld", a.nchunks, 0), hipErrorInvalidValue;
  if (a.identity && (a.log2d != 4 || a.signs || a.scale != 1.0f || a.mode != RH_QUANT))
    return violation("quantize-only launch with a transform (log2 d %lld, mode %lld)", a.log2d, a.mode), hipErrorInvalidValue;
  if (l2d < 4 || l2d > 12 || a.n % d || a.cpr != a.n / d || a.nchunks != a.rows * a.cpr)
    return violation("row Hadamard shape (d %lld, n %lld)", d, a.n), hipErrorInvalidValue;
  {  // the rounds' new bits partition the index bits; each round's layout is a bijection
    unsigned done = 0;
    for (int r = 0; r < R; ++r)
      for (int q = 4 - rh_nnew(l2d, r); q < 4; ++q) {
        const int bit = rh_regbit(l2d, r, q);
        if (bit < 4 * r || bit >= l2d || ((done >> bit) & 1))
          return violation("round %lld transforms bit %lld twice or out of range", r, bit), hipErrorInvalidValue;
        done |= 1u << bit;
      }
    if (done != (l2d == 32 ? ~0u : (1u << l2d) - 1))
      return violation("rounds leave bits untransformed", 0, 0), hipErrorInvalidValue;
    for (int r = 0; r < R; ++r) {
      std::vector<uint8_t> seen(d, 0);
      for (int cu = 0; cu < d / 16; ++cu)
        for (int j = 0; j < 16; ++j) {
          const int e = rh_elem(l2d, r, cu, j);
          if (e < 0 || e >= d || seen[e]++) return violation("round %lld layout is not a bijection (%lld)", r, e), hipErrorInvalidValue;
          for (int q = 0; q < 4; ++q)
            if (((e >> rh_regbit(l2d, r, q)) & 1) != ((j >> q) & 1))
              return violation("register bit %lld of round %lld", q, r), hipErrorInvalidValue;
        }
      for (int cu = 0; cu < d / 16; ++cu)
        for (int j = 0; j < 16; ++j)
          if (rh_elem(l2d, 0, cu, j) != 16 * cu + j)
            return violation("round 0 is not natural order (%lld, %lld)", cu, j), hipErrorInvalidValue;
    }
    // the kernel's split addressing: per-thread base + per-register constant
    for (int r = 0; r < R; ++r)
      for (int u = 0; u < kRhThreads; ++u) {
        const int cw = u >> (l2d - 4), cu = u & ((1 << (l2d - 4)) - 1);
        for (int j = 0; j < 16; ++j)
          if (rh_lds_base(l2d, r, cw, cu) + rh_lds_off(l2d, r, j) != rh_lds(l2d, cw, rh_elem(l2d, r, cu, j)))
            return violation("split LDS address of thread %lld, round %lld", u, r), hipErrorInvalidValue;
      }
    std::vector<int> slot(kRhLds);
    for (int r = 0; r < R && R > 1; ++r) {
      std::fill(slot.begin(), slot.end(), -1);
      for (int u = 0; u < kRhThreads; ++u) {
        const int cw = u >> (l2d - 4), cu = u & ((1 << (l2d - 4)) - 1);
        for (int j = 0; j < 16; ++j) {
          const int e = rh_elem(l2d, r, cu, j);
          const int s = rh_lds(l2d, cw, e);
          if (s < 0 || s >= kRhLds || slot[s] != -1) return violation("LDS slot %lld written twice", s, r), hipErrorInvalidValue;
          slot[s] = (cw << l2d) + e;
        }
      }
      const int rn = r + 1 < R ? r + 1 : 0;
      for (int u = 0; u < kRhThreads; ++u) {
        const int cw = u >> (l2d - 4), cu = u & ((1 << (l2d - 4)) - 1);
        for (int j = 0; j < 16; ++j) {
          const int e = rh_elem(l2d, rn, cu, j);
          const int s = rh_lds(l2d, cw, e);
          if (s < 0 || s >= kRhLds || slot[s] != (cw << l2d) + e)
            return violation("LDS read of slot %lld in round %lld", s, r), hipErrorInvalidValue;
        }
      }
    }
  }
  if (a.mode == RH_QUANT && a.qkind == BRQ_CODEBOOK_NORM && a.bin_s != 0.f) {
    // the codebook bins: each threshold alone in a bin strictly inside the clamp range
    int prev = 0;
    for (int k = 0; k + 1 < a.nlev; ++k) {
      const int b = rh_bin(std::fma(a.tau[k], a.bin_s, a.bin_off));
      if (b <= prev || b >= kRhBins - 1)
        return violation("codebook threshold %lld in bin %lld", k, b), hipErrorInvalidValue;
      if (a.tbin[k] != b) return violation("threshold %lld recorded in bin %lld", k, a.tbin[k]), hipErrorInvalidValue;
      int cnt;
      std::memcpy(&cnt, &a.bintab[b].y, sizeof cnt);
      if (a.bintab[b].x != std::fma(a.tau[k], a.bin_s, a.bin_off) || cnt != k)
        return violation("bin table entry %lld (threshold %lld)", b, k), hipErrorInvalidValue;
      prev = b;
    }
    if (a.nlev - 1 > kMaxLevels || a.nlev > kRhThreads)
      return violation("codebook of %lld levels", a.nlev, 0), hipErrorInvalidValue;
  }
  const int64_t nwg = rh_nwg(a);
  const int esz_x = a.xt == BRQ_F32 ? 4 : 2, esz_y = a.yt == BRQ_F32 ? 4 : 2;
  const bool deq = a.mode == RH_DEQUANT || a.mode == RH_REQUANT;
  const bool qout = a.mode == RH_QUANT || a.mode == RH_REQUANT;
  if (a.mode == RH_REQUANT && (l2d < 6 || l2d > 8 || a.bits2 < 2 || a.bits2 > 5 || !a.inverse ||
                               a.h2 != (float)(((1 << a.bits2) - 1) * 0.5)))
    return violation("re-quantizer launch (log2 d %lld, bits %lld)", l2d, a.bits2), hipErrorInvalidValue;
  // the output quantizer's width, group and row strides
  const int obits = a.mode == RH_REQUANT ? a.bits2 : a.bits;
  const int ogroup = a.mode == RH_REQUANT ? a.group2 : a.group;
  const int64_t ocodes_ld = a.mode == RH_REQUANT ? a.codes_ld2 : a.codes_ld;
  const int64_t oscales_ld = a.mode == RH_REQUANT ? a.scales_ld2 : a.scales_ld;
  std::vector<uint8_t> cover((size_t)(a.rows * a.n), 0);
  std::vector<uint8_t> scov;
  if (qout) scov.assign((size_t)(a.rows * oscales_ld), 0);
  const int lpg = qout ? ogroup / 16 : 1;
  if (qout && (ogroup % 16 || lpg > 64 || (lpg & (lpg - 1)) || kRhTile % ogroup))
    return violation("quantizer group %lld", ogroup, 0), hipErrorInvalidValue;
  if (deq && (a.group % 16 || a.group < 16))
    return violation("dequantizer group %lld", a.group, 0), hipErrorInvalidValue;
  for (int64_t b = 0; b < nwg; ++b)
    for (int u = 0; u < kRhThreads; ++u) {
      const RhPos p = rh_pos(a, b, u);
      if (!p.live) {  // dead threads read the first 16 elements of row 0
        if (p.row != 0 || p.col0 != 0) return violation("dead thread %lld reads (%lld)", u, p.row), hipErrorInvalidValue;
        continue;
      }
      if (p.row >= a.rows || p.col0 < 0 || p.col0 + 16 > a.n || p.col0 % 16)
        return violation("row Hadamard element (%lld, %lld)", p.row, p.col0), hipErrorInvalidValue;
      if (p.col0 % d != 16 * p.cu) return violation("chunk position of thread %lld", u, 0), hipErrorInvalidValue;
      if (!deq) {
        const int64_t off = p.row * a.ldx + p.col0;
        if (p.col0 + 16 > a.ldx || (off * esz_x) % 16) return violation("row Hadamard load %lld", off, 0), hipErrorInvalidValue;
      } else {
        const int64_t off = p.row * a.codes_ld + p.col0 * a.bits / 8;
        if (!in_range(off, 2 * a.bits, a.rows * a.codes_ld) || off % ((a.bits & 1) ? 2 : 4))
          return violation("code read at %lld", off, 0), hipErrorInvalidValue;
        if (!in_range(p.row * a.scales_ld + p.col0 / a.group, 1, a.rows * a.scales_ld))
          return violation("scale read (%lld, %lld)", p.row, p.col0), hipErrorInvalidValue;
      }
      if (!qout) {
        const int64_t off = p.row * a.ldy + p.col0;
        if (p.col0 + 16 > a.ldy || (off * esz_y) % 16) return violation("row Hadamard store %lld", off, 0), hipErrorInvalidValue;
      } else {
        const int64_t off = p.row * ocodes_ld + p.col0 * obits / 8;
        if (!in_range(off, 2 * obits, a.rows * ocodes_ld) || off % ((obits & 1) ? 2 : 4))
          return violation("code write at %lld", off, 0), hipErrorInvalidValue;
        if (u % lpg == 0) {  // the group's lanes: same wave, same row, contiguous columns
          if (p.col0 % ogroup) return violation("group start column %lld", p.col0, 0), hipErrorInvalidValue;
          for (int k = 1; k < lpg; ++k) {
            const RhPos o = rh_pos(a, b, u + k);
            if ((u + k) / 64 != u / 64 || !o.live || o.row != p.row || o.col0 != p.col0 + 16 * k)
              return violation("group lanes of thread %lld (lane +%lld)", u, k), hipErrorInvalidValue;
          }
          const int64_t sidx = p.row * oscales_ld + p.col0 / ogroup;
          if (!in_range(sidx, 1, a.rows * oscales_ld) || scov[(size_t)sidx]++)
            return violation("scale %lld written twice or out of range", sidx, 0), hipErrorInvalidValue;
        }
      }
      for (int j = 0; j < 16; ++j) cover[(size_t)(p.row * a.n + p.col0 + j)]++;
    }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return violation("row Hadamard element %lld covered %lld times", (int64_t)i, cover[i]), hipErrorInvalidValue;
  for (size_t i = 0; i < scov.size(); ++i)
    if (scov[i] != 1) return violation("scale %lld written %lld times", (int64_t)i, scov[i]), hipErrorInvalidValue;
  return hipSuccess;
}

}  // namespace brq

// ---------------------------------------------------------------- stage pass

#include "stage.h"

namespace brq {

hipError_t launch_stage(const SpArgs& a, hipStream_t) {
  ++g_launches;
  const int b = a.b;
  if ((a.tile_lines != 0 && (a.side != 0 || (a.tile_lines != kSpLinesFew && a.tile_lines != kSpLinesTiny))) ||
      b < 2 || b > 64 || a.bp < b || (a.bp & (a.bp - 1)) || a.bp > 64 || a.bs < b || a.bs % 4 ||
      a.bs - b >= 4 || a.gw < 1 || a.gw * a.bp > kSpThreads || a.gw * a.bs > kSpLineFloats)
    return violation("stage pass geometry (b %lld, gw %lld)", b, a.gw), hipErrorInvalidValue;
  if (a.S < 1 || a.d % (b * a.S) || a.ngc != a.d / b || a.ngroups % a.ngc)
    return violation("stage pass shape (d %lld, S %lld)", a.d, a.S), hipErrorInvalidValue;
  if (a.mode == BRQ_HADAMARD ? (a.blk || (b & (b - 1))) : !a.blk)
    return violation("stage pass blocks (mode %lld)", a.mode, 0), hipErrorInvalidValue;
  const int64_t nchunk = a.ngroups / a.ngc;
  const int64_t axis_len = nchunk * a.d;  // positions along the transformed axis
  if (axis_len >= ((int64_t)1 << 31)) return violation("positions beyond 32 bits (%lld)", axis_len, 0), hipErrorInvalidValue;
  const int64_t rows = a.side == 0 ? a.lines : axis_len;
  const int64_t cols = a.side == 0 ? axis_len : a.lines;
  if (a.ld_src < cols || a.ld_dst < cols)
    return violation("stage pass leading dimension (%lld < %lld)", std::min(a.ld_src, a.ld_dst), cols), hipErrorInvalidValue;
  const int64_t nblocks = sp_blocks(a);
  if (nblocks >= ((int64_t)1 << 31)) return violation("stage pass grid (%lld blocks)", nblocks, 0), hipErrorInvalidValue;
  // a source of several parts: right side, float32, parts no closer than one
  // whole source apart (every read of part p is the part-0 read plus p strides)
  if (a.nparts > 1 && (a.side != 0 || a.src_t != BRQ_F32 || a.part_stride < rows * a.ld_src))
    return violation("stage pass parts (%lld parts, stride %lld)", a.nparts, a.part_stride), hipErrorInvalidValue;
  const int64_t blk_floats = a.mode == BRQ_PER_GROUP ? a.ngc * b * b : (int64_t)b * b;
  const int TL = sp_tl(a);
  const int kLds = a.side ? kSpBufFloats : TL * kSpLineFloats;
  std::vector<uint8_t> cover((size_t)(rows * cols), 0);
  std::vector<int> xin(kLds), yout(kLds);
  std::vector<uint8_t> tile_seen((size_t)(sp_group_tiles(a) * sp_line_tiles(a)), 0);
  for (int64_t bid = 0; bid < nblocks; ++bid) {
      int64_t gt, lt;
      sp_tile_of_block(a, (uint32_t)bid, gt, lt);
      if (gt < 0 || gt >= sp_group_tiles(a) || lt < 0 || lt >= sp_line_tiles(a) ||
          tile_seen[(size_t)(gt * sp_line_tiles(a) + lt)]++)
        return violation("stage pass block %lld maps to a bad or repeated tile (%lld)", bid, gt), hipErrorInvalidValue;
      const int64_t g0 = gt * a.gw, l0 = lt * TL;
      const int ng = (int)std::min<int64_t>(a.ngroups - g0, a.gw);
      const int nl = (int)std::min<int64_t>(a.lines - l0, TL);
      const int gb = a.gw * b;
      std::fill(xin.begin(), xin.end(), 0);
      std::fill(yout.begin(), yout.end(), 0);
      // block rows
      for (int u = 0; u < kSpThreads; ++u) {
        const int g = u / a.bp, j = u - g * a.bp;
        if (j >= b || g >= ng || a.mode == BRQ_HADAMARD) continue;
        const int64_t r = sp_block_row(a, g0 + g, j);
        if (r < 0 || r + b > blk_floats) return violation("block row at %lld of %lld", r, blk_floats), hipErrorInvalidValue;
        if (a.mode == BRQ_PER_GROUP && r / (b * b) != ((g0 + g) % a.ngc))
          return violation("block of group %lld read at %lld", g0 + g, r), hipErrorInvalidValue;
        if (a.blk_vec && (b % 4 || r % 4 || reinterpret_cast<uintptr_t>(a.blk) % 16))
          return violation("vector block row at %lld (b %lld)", r, b), hipErrorInvalidValue;
      }
      // padding
      for (int e = 0; e < TL * a.gw; ++e) {
        const int l = e / a.gw, gg = e - l * a.gw;
        for (int k = b; k < a.bs; ++k) {
          const int s = sp_lds(a, l, gg, k);
          if (s < 0 || s >= kLds) return violation("LDS pad slot %lld", s, 0), hipErrorInvalidValue;
          xin[s] = 1;
        }
      }
      // the (g, k) members each load/store thread takes, and the lines it walks
      auto members = [&](auto&& fn) -> bool {
        if (a.side == 0) {
          for (int u = 0; u < kSpThreads && u < gb; ++u) {
            int gg, k;
            sp_member(a, u, gg, k);
            if (gg < ng)
              for (int l = 0; l < nl; ++l)
                if (!fn(l, gg, k)) return false;
          }
        } else {
          if (gb > kSpLines * (kSpThreads / kSpLines))
            return violation("left-side tile of %lld members exceeds the unrolled loads", gb, 0);
          for (int u = 0; u < kSpThreads; ++u) {
            const int l = u % kSpLines;
            for (int q = u / kSpLines; q < gb; q += kSpThreads / kSpLines) {
              int gg, k;
              sp_member(a, q, gg, k);
              if (gg < ng && l < nl && !fn(l, gg, k)) return false;
            }
          }
        }
        return true;
      };
      bool ok = members([&](int l, int gg, int k) {
        if (k < 0 || k >= b || gg < 0 || gg >= a.gw) return violation("member (%lld, %lld)", gg, k);
        const int64_t pos = sp_pos(a, g0 + gg, k);
        if (pos < 0 || pos >= axis_len) return violation("position %lld of %lld", pos, axis_len);
        const int64_t off = sp_off(a, l0 + l, pos, a.ld_src);
        const int64_t line = l0 + l;
        if (line >= a.lines || off < 0 || off >= (a.side == 0 ? rows * a.ld_src : axis_len * a.ld_src))
          return violation("stage pass load at %lld (line %lld)", off, line);
        const int s = sp_lds(a, l, gg, k);
        if (s != sp_lds(a, l, 0, 0) + sp_lds(a, 0, gg, k)) return violation("LDS slot split at %lld", s, 0);
        if (a.side == 1 && pos >= a.d) return violation("left-side sign index %lld", pos, a.d);
        if (s < 0 || s >= kLds || xin[s]) return violation("LDS slot %lld loaded twice", s, 0);
        xin[s] = 1;
        return true;
      });
      if (!ok) return hipErrorInvalidValue;
      // compute: thread (g, j) reads slots k < bs of its group for each line, writes slot j
      for (int u = 0; u < kSpThreads; ++u) {
        const int g = u / a.bp, j = u - g * a.bp;
        if (j >= b || g >= ng) continue;
        if (a.side == 1)  // float4 over lines 4 l4 .. 4 l4 + 3 (those past nl are discarded)
          for (int l4 = 0; 4 * l4 < nl; ++l4)
            for (int k = 0; k < b; ++k) {
              const int base = sp_lds(a, 4 * l4, g, k);
              if (base % 4 || base + 4 > kLds) return violation("left-side LDS vector read at %lld", base, 0), hipErrorInvalidValue;
              for (int i = 0; i < 4 && 4 * l4 + i < nl; ++i)
                if (!xin[base + i]) return violation("LDS read of unwritten slot %lld", base + i, 0), hipErrorInvalidValue;
            }
        for (int l = 0; l < nl; ++l) {
          const int base = sp_lds(a, l, g, 0);
          if (a.side == 0) {
            if (base % 4) return violation("unaligned LDS vector read at %lld", base, 0), hipErrorInvalidValue;
            for (int k = 0; k < a.bs; ++k)
              if (base + k >= kLds || !xin[base + k]) return violation("LDS read of unwritten slot %lld", base + k, 0), hipErrorInvalidValue;
          }
          const int s = a.b2 && !a.inv2 ? sp_lds(a, l, j, g) : sp_lds(a, l, g, j);
          if (yout[s]++) return violation("LDS output slot %lld written twice", s, 0), hipErrorInvalidValue;
        }
      }
      if (a.b2) {  // the second stage: reads (g2, k2) (forward) or (k2, g2) (inverse), writes (j2, g2)
        if (a.side != 0 || a.gw != 16 || a.S != (a.inv2 ? 1 : 16) || a.b != 16 || a.b2 != 16 || a.bs != 16 || a.bp != 16 ||
            ng != a.gw || (a.mode != BRQ_HADAMARD && (!a.blk2 || reinterpret_cast<uintptr_t>(a.blk2) % 16)))
          return violation("stage pair geometry (b %lld, b2 %lld)", a.b, a.b2), hipErrorInvalidValue;
        const int64_t blk2_floats = a.mode == BRQ_PER_GROUP ? (a.d / a.b2) * a.b2 * a.b2 : (int64_t)a.b2 * a.b2;
        for (int u = 0; u < kSpThreads; ++u) {
          const int g2 = u / a.b2, j2 = u - g2 * a.b2;
          if (g2 >= a.b || j2 >= a.b2) continue;
          if (a.mode != BRQ_HADAMARD) {
            const int64_t r = sp_block_row2(a, g0, g2, j2);
            if (r < 0 || r + a.b2 > blk2_floats) return violation("second-stage block row %lld of %lld", r, blk2_floats), hipErrorInvalidValue;
          }
          for (int l = 0; l < nl; ++l) {  // the first stage wrote (j, g) = every slot of the block
            for (int k2 = 0; k2 < a.b2; ++k2) {
              const int sr = a.inv2 ? sp_lds(a, l, k2, g2) : sp_lds(a, l, g2, k2);
              if (a.inv2 && sr != sp_lds(a, l, 0, g2) + 16 * k2) return violation("second stage column read at %lld", sr, 0), hipErrorInvalidValue;
              if (yout[sr] != 1) return violation("second stage reads slot %lld", sr, 0), hipErrorInvalidValue;
            }
            if (!a.inv2 && sp_lds(a, l, g2, 0) % 4) return violation("second stage vector read at %lld", sp_lds(a, l, g2, 0), 0), hipErrorInvalidValue;
            if (yout[sp_lds(a, l, j2, g2)] != 1) return violation("second stage writes slot %lld", sp_lds(a, l, j2, g2), 0), hipErrorInvalidValue;
          }
        }
      }
      ok = members([&](int l, int gg, int k) {
        const int s = sp_lds(a, l, gg, k);
        if (yout[s] != 1) return violation("LDS output slot %lld read before it is written", s, 0);
        const int64_t pos = sp_pos(a, g0 + gg, k);
        const int64_t r = a.side == 0 ? l0 + l : pos, c = a.side == 0 ? pos : l0 + l;
        if (r >= rows || c >= cols) return violation("stage pass store (%lld, %lld)", r, c);
        if (sp_off(a, l0 + l, pos, a.ld_dst) != r * a.ld_dst + c) return violation("store offset of (%lld, %lld)", r, c);
        cover[(size_t)(r * cols + c)]++;
        return true;
      });
      if (!ok) return hipErrorInvalidValue;
    }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return violation("stage pass element %lld stored %lld times", (int64_t)i, cover[i]), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_stage_rows(const SpArgs& a, hipStream_t) {
  ++g_launches;
  ++g_rows_launches;
  const int b = a.b;
  if (!sr_supported(a)) return violation("rows kernel launched for an unsupported stage (b %lld)", b, 0), hipErrorInvalidValue;
  if (a.S < 1 || a.d % (b * a.S) || a.ngc != a.d / b || a.ngroups != a.ngc)
    return violation("rows kernel shape (d %lld, S %lld)", a.d, a.S), hipErrorInvalidValue;
  const int vec = sr_vec(b);
  const int64_t rows = a.d, cols = a.lines;
  if (a.ld_src < cols || a.ld_dst < cols)
    return violation("rows kernel leading dimension (%lld < %lld)", std::min(a.ld_src, a.ld_dst), cols), hipErrorInvalidValue;
  const int64_t nct = sr_col_tiles(a), nblk = nct * a.ngroups;
  if (nblk >= ((int64_t)1 << 31) || nct * kSrThreads * vec < cols)
    return violation("rows kernel grid (%lld blocks, %lld column tiles)", nblk, nct), hipErrorInvalidValue;
  const int64_t blk_floats = a.mode == BRQ_PER_GROUP ? a.ngc * b * b : (int64_t)b * b;
  std::vector<uint8_t> loaded((size_t)(rows * cols), 0), stored((size_t)(rows * cols), 0);
  for (int64_t bid = 0; bid < nblk; ++bid) {
    uint32_t gid, ct;
    sr_tile_of_block((uint32_t)bid, (uint32_t)nct, gid, ct);
    if (gid >= a.ngroups || ct >= nct) return violation("rows kernel block %lld maps to group %lld", bid, gid), hipErrorInvalidValue;
    if (a.mode != BRQ_HADAMARD) {
      const int64_t r = sp_block_row(a, gid, 0);
      if (r < 0 || r + (int64_t)b * b > blk_floats) return violation("rows kernel block at %lld of %lld", r, blk_floats), hipErrorInvalidValue;
      if (a.mode == BRQ_PER_GROUP && r != (int64_t)gid * b * b) return violation("block of group %lld read at %lld", gid, r), hipErrorInvalidValue;
    }
    for (int t = 0; t < kSrThreads; ++t) {
      const int64_t c0 = sr_col(ct, t, vec);
      if (c0 >= cols) continue;
      if (c0 + vec > cols || c0 % vec) return violation("rows kernel vector at column %lld", c0, 0), hipErrorInvalidValue;
      for (int k = 0; k < b; ++k) {
        const int64_t row = sp_pos(a, gid, k);
        if (row < 0 || row >= rows) return violation("rows kernel row %lld of %lld", row, rows), hipErrorInvalidValue;
        if (row != ((int64_t)gid / a.S) * b * a.S + (int64_t)k * a.S + gid % a.S)
          return violation("member %lld of group %lld at the wrong row", k, gid), hipErrorInvalidValue;
        for (int v = 0; v < vec && c0 + v < cols; ++v) {
          const int64_t e = row * cols + c0 + v;
          if (loaded[(size_t)e]++) return violation("rows kernel loads (%lld, %lld) twice", row, c0 + v), hipErrorInvalidValue;
          if (stored[(size_t)e]++) return violation("rows kernel stores (%lld, %lld) twice", row, c0 + v), hipErrorInvalidValue;
        }
      }
    }
  }
  for (size_t i = 0; i < stored.size(); ++i)
    if (stored[i] != 1) return violation("rows kernel element %lld stored %lld times", (int64_t)i, stored[i]), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_harp(const HarpArgs& a, hipStream_t) {
  ++g_launches;
  if (a.b < 2 || a.b > 64 || a.np != harp_params(a.b) || a.ngroups < 0 || a.ngroups >= ((int64_t)1 << 31))
    return violation("HARP launch geometry (b %lld, ngroups %lld)", a.b, a.ngroups), hipErrorInvalidValue;
  if (!a.base && (a.b & (a.b - 1))) return violation("HARP radix %lld without a base mixer", a.b, 0), hipErrorInvalidValue;
  const int b = a.b, P = harp_pitch(b);
  if (harp_lds_bytes(b) > 160 * 1024) return violation("HARP LDS %lld bytes", (long long)harp_lds_bytes(b), 0), hipErrorInvalidValue;
  // one block: every parameter index in range and used once per (i < j), LDS
  // slots within the system, outputs once each
  std::vector<int> used(a.np, 0);
  if (b == 2) {
    used[0] = 1;
  } else {
    for (int i = 0; i < b; ++i)
      for (int j = 0; j < b; ++j) {
        if (i * P + b + j >= b * P) return violation("HARP LDS slot (%lld, %lld)", i, j), hipErrorInvalidValue;
        if (i < j) {
          const int p = harp_pidx(b, i, j);
          if (p < 0 || p >= a.np || used[p]++) return violation("HARP parameter index %lld (b %lld)", p, b), hipErrorInvalidValue;
        }
      }
  }
  for (int p = 0; p < a.np; ++p)
    if (used[p] != 1) return violation("HARP parameter %lld unused", p, 0), hipErrorInvalidValue;
  if (2 * b > 2 * kHpThreads) return violation("HARP columns per lane (b %lld)", b, 0), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_harp_batch(const HarpBatch& a, hipStream_t s) {
  if (a.n < 1 || a.n > kHpMaxJobs || a.first[0] != 0)
    return violation("HARP batch of %lld jobs", a.n, 0), hipErrorInvalidValue;
  for (int j = 0; j < a.n; ++j) {
    const HarpArgs& h = a.job[j];
    if (!harp_batchable(h.b) || h.ngroups < 1 || a.first[j + 1] != a.first[j] + h.ngroups)
      return violation("HARP batch job %lld (b %lld)", j, h.b), hipErrorInvalidValue;
    const hipError_t e = launch_harp(h, s);  // the per-block checks
    --g_launches;
    if (e != hipSuccess) return e;
    for (int k = 0; k < j; ++k) {  // outputs of distinct jobs do not overlap
      const HarpArgs& o = a.job[k];
      const float *lo1 = h.out, *hi1 = h.out + h.ngroups * h.b * h.b;
      const float *lo2 = o.out, *hi2 = o.out + o.ngroups * o.b * o.b;
      if (lo1 < hi2 && lo2 < hi1) return violation("HARP batch outputs %lld and %lld overlap", k, j), hipErrorInvalidValue;
    }
  }
  if (a.first[a.n] >= ((int64_t)1 << 31)) return violation("HARP batch grid %lld", a.first[a.n], 0), hipErrorInvalidValue;
  // every workgroup finds its job: the scan the kernel does
  for (int64_t w : {(int64_t)0, a.first[a.n] - 1}) {
    int j = 0;
    while (j + 1 < a.n && w >= a.first[j + 1]) ++j;
    if (w < a.first[j] || w >= a.first[j + 1]) return violation("HARP batch block %lld", w, 0), hipErrorInvalidValue;
  }
  ++g_launches;
  ++g_harp_batches;
  return hipSuccess;
}

hipError_t launch_stage_pair2(const P2Args& a, hipStream_t) {
  ++g_launches;
  ++g_pair2_launches;
  const int n = a.bo * a.bi;
  if (a.bo < 2 || a.bi < 2 || a.bo > 16 || a.bi > 16 || n > 256 || a.sets > 256 / n || a.sets < 1 ||
      a.lines < 1 || a.lines > kP2MaxLines || a.Si < 1 || a.d % (n * a.Si))
    return violation("stage pair geometry (bo %lld, bi %lld)", a.bo, a.bi), hipErrorInvalidValue;
  const int64_t per_chunk = a.d / (n * a.Si) * a.Si;
  if (a.nsets % per_chunk || a.ld_src < a.nsets / per_chunk * a.d || a.ld_dst < a.nsets / per_chunk * a.d)
    return violation("stage pair sets %lld (chunk %lld)", a.nsets, per_chunk), hipErrorInvalidValue;
  const int64_t cols = a.nsets / per_chunk * a.d;
  const int64_t blk_o = a.per_group ? a.d / a.bo * a.bo * a.bo : a.bo * a.bo;
  const int64_t blk_i = a.per_group ? a.d / a.bi * a.bi * a.bi : a.bi * a.bi;
  std::vector<uint8_t> seen((size_t)(cols * a.lines), 0);
  const int64_t nb = p2_blocks(a), nsb = p2_set_blocks(a);
  if (nb >= ((int64_t)1 << 31)) return violation("stage pair grid %lld", nb, 0), hipErrorInvalidValue;
  for (int64_t blk = 0; blk < nb; ++blk)
    for (int u = 0; u < 256; ++u) {
      const int sl = u / n, e = u - sl * n;
      int64_t sbk, lb;
      p2_tile(a, blk, sbk, lb);
      if (sbk < 0 || sbk >= nsb || lb < 0 || lb * nsb + sbk >= nb)
        return violation("stage pair workgroup %lld maps to (%lld, ...)", blk, sbk), hipErrorInvalidValue;
      const int64_t s = sbk * a.sets + sl, l0 = lb * kP2Lines;
      const int nl = (int)std::min<int64_t>(a.lines - l0, kP2Lines);
      if (sl >= a.sets || s >= a.nsets) continue;
      if (nl < 1) return violation("stage pair line tile at %lld", l0, 0), hipErrorInvalidValue;
      int64_t c, hi, lo;
      p2_set(a, s, c, hi, lo);
      const int ea = e / a.bi, eb = e - ea * a.bi, og = e / a.bo, oj = e - og * a.bo;
      const int64_t pos = p2_pos(a, c, hi, lo, ea, eb);
      if (pos < 0 || pos >= cols) return violation("stage pair position %lld", pos, 0), hipErrorInvalidValue;
      for (int l = 0; l < nl; ++l)
        if (seen[(size_t)((l0 + l) * cols + pos)]++) return violation("stage pair element (%lld, %lld)", l0 + l, pos), hipErrorInvalidValue;
      if (pos / a.d != c) return violation("stage pair chunk of %lld", pos, 0), hipErrorInvalidValue;
      const int64_t ro = p2_row_o(a, hi, lo, og, oj), ri = p2_row_i(a, hi, lo, ea, eb);
      if (ro < 0 || ro + a.bo > blk_o || ri < 0 || ri + a.bi > blk_i)
        return violation("stage pair block rows %lld, %lld", ro, ri), hipErrorInvalidValue;
      if (a.vec_i && (a.bi % 4 || ri % 4 || reinterpret_cast<uintptr_t>(a.blk_i) % 16))
        return violation("stage pair vector block row at %lld (bi %lld)", ri, a.bi), hipErrorInvalidValue;
      // the outer group og mixes positions (k, og), the inner group ea positions (ea, k): same chunk, hi, lo
      for (int k = 0; k < a.bo; ++k)
        if (p2_pos(a, c, hi, lo, k, og) / (n * a.Si) != pos / (n * a.Si)) return violation("stage pair set %lld", s, 0), hipErrorInvalidValue;
      const int lds_max = (sl + 1) * kP2Lines * n;
      if (lds_max > 256 * kP2Lines) return violation("stage pair LDS %lld", lds_max, 0), hipErrorInvalidValue;
    }
  for (size_t i = 0; i < seen.size(); ++i)
    if (seen[i] != 1) return violation("stage pair position %lld covered %lld times", (int64_t)i, seen[i]), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_stage_lanes(const SpArgs& a, int rows_per, hipStream_t) {
  ++g_launches;
  ++g_lanes_launches;
  const int b = a.b;
  if (!sl_supported(a) || rows_per != sl_rows_per(a) || (b <= 8 && (rows_per % 4 || rows_per < 4)))
    return violation("lanes kernel launched for an unsupported stage (b %lld, rows %lld)", b, rows_per), hipErrorInvalidValue;
  if (a.S < 1 || a.d % (b * a.S) || a.ngc != a.d / b || a.ngroups % a.ngc)
    return violation("lanes kernel shape (d %lld, S %lld)", a.d, a.S), hipErrorInvalidValue;
  const int64_t nchunk = a.ngroups / a.ngc, axis = nchunk * a.d, rows = a.lines;
  if (axis >= ((int64_t)1 << 31)) return violation("positions beyond 32 bits (%lld)", axis, 0), hipErrorInvalidValue;
  if (a.ld_src < axis || a.ld_dst < axis)
    return violation("lanes kernel leading dimension (%lld < %lld)", std::min(a.ld_src, a.ld_dst), axis), hipErrorInvalidValue;
  const SlGeom g = sl_geom(a, rows_per);
  const int64_t blk_floats = a.mode == BRQ_PER_GROUP ? a.ngc * b * b : (int64_t)b * b;
  std::vector<uint8_t> cover((size_t)(rows * axis), 0);
  for (int64_t bid = 0; bid < g.lo_tiles * g.row_tiles; ++bid) {
    const int64_t t = bid % g.lo_tiles, rt = bid / g.lo_tiles;
    // the tile's 64 groups: one chunk, one hi, consecutive lo
    const int64_t g0 = sl_group(t, 0);
    if (g0 / a.ngc != (g0 + kSlLanes - 1) / a.ngc || ((g0 % a.ngc) / a.S) != (((g0 + kSlLanes - 1) % a.ngc) / a.S))
      return violation("lane tile %lld spans chunks or strides", t, 0), hipErrorInvalidValue;
    if (a.mode == BRQ_PER_GROUP) {
      const int64_t base = sp_block_row(a, g0, 0);
      if (base < 0 || base + (int64_t)kSlLanes * b * b > blk_floats)
        return violation("lane tile blocks at %lld of %lld", base, blk_floats), hipErrorInvalidValue;
      for (int l = 0; l < kSlLanes; ++l)
        if (sp_block_row(a, sl_group(t, l), 0) != base + (int64_t)l * b * b)
          return violation("blocks of lane %lld are not contiguous", l, 0), hipErrorInvalidValue;
    }
    for (int l = 0; l < kSlLanes; ++l) {
      const int64_t gid = sl_group(t, l);
      const int64_t pos0 = sp_pos(a, gid, 0);
      for (int k = 0; k < b; ++k) {
        const int64_t pos = pos0 + (int64_t)k * a.S;
        if (pos != sp_pos(a, gid, k) || pos < 0 || pos >= axis)
          return violation("lane member position %lld (k %lld)", pos, k), hipErrorInvalidValue;
        if ((uint32_t)(pos0 % a.d) + (uint32_t)(k * a.S) >= (uint32_t)a.d)
          return violation("lane sign index beyond d (%lld)", pos, 0), hipErrorInvalidValue;
        // radix <= 8: wave w stores every output of rows w, w + 4, ...;
        // radix 16: wave k / 4 stores output k of every row
        for (int w = 0; w < kSlThreads / kSlLanes; ++w) {
          if (b == 16 && w != k / 4) continue;
          const int step = b == 16 ? 1 : 4;
          for (int64_t r = rt * rows_per + (b == 16 ? 0 : w); r < std::min(rt * rows_per + rows_per, rows); r += step)
            if (cover[(size_t)(r * axis + pos)]++)
              return violation("lanes kernel element (%lld, %lld) twice", r, pos), hipErrorInvalidValue;
        }
        if (b == 16 && a.mode != BRQ_HADAMARD &&
            (sp_block_row(a, gid, 4 * (k / 4)) % 4 || reinterpret_cast<uintptr_t>(a.blk) % 16))
          return violation("radix-16 block rows of group %lld not 16-byte aligned", gid, 0), hipErrorInvalidValue;
      }
    }
  }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return violation("lanes kernel element %lld covered %lld times", (int64_t)i, cover[i]), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_qlinear(const QlArgs& a, hipStream_t) {
  ++g_launches;
  const int TN = a.tn;
  if (a.kind != ql_kind(a.T, a.m, a.n, a.bits, a.group, reinterpret_cast<uintptr_t>(a.codes) % 16 == 0) ||
      TN != ql_kind_tn(a.kind, a.tm) || a.tv != (int)std::min<int64_t>(a.T, (int64_t)kQlTok * a.tm))
    return violation("quantized linear kernel choice (kind %lld, tn %lld)", a.kind, TN), hipErrorInvalidValue;
  if (a.bits < 2 || a.bits > 5 || (a.group != 64 && a.group != 128) || a.n % a.group || a.m % (kQlOut * TN) ||
      a.kc % a.group || a.kc <= 0 || a.splits < 1 || (a.splits - 1) * a.kc >= a.n || a.splits * a.kc < a.n ||
      a.tm != ql_kind_tm(a.kind, a.T, a.bits, a.group))
    return violation("quantized linear geometry (splits %lld, kc %lld)", a.splits, a.kc), hipErrorInvalidValue;
  if (a.ldx < a.n || a.ldx % 8 || reinterpret_cast<uintptr_t>(a.x) % 16)
    return violation("activation rows not 16-byte vectors (ld %lld)", a.ldx, 0), hipErrorInvalidValue;
  if (a.codes_ld != a.n * a.bits / 8 || a.scales_ld != a.n / a.group)
    return violation("code or scale row length %lld", a.codes_ld, 0), hipErrorInvalidValue;
  const int64_t nb = ql_blocks(a);
  if (nb >= ((int64_t)1 << 31)) return violation("quantized linear grid %lld", nb, 0), hipErrorInvalidValue;
  const int NC = a.group / 4, NB = NC * a.bits / 8;
  if (a.kind != kQlDirect) {  // whole chunks per split, 16-byte rows, and the LDS the launch asks for
    const bool gemm = a.kind == kQlGemm;
    const int CK = gemm ? kQlGemmChunk : kQlChunk;
    const int R = kQlOut * TN, CB = CK * a.bits / 8, PB = ql_code_pitch_ck(a.bits, CK);
    const int tv = a.tv;
    const size_t lds_cap = gemm ? 160 * 1024 : 64 * 1024;
    if (a.n % CK || a.kc % CK || reinterpret_cast<uintptr_t>(a.codes) % 16 || a.codes_ld % 16 ||
        ql_lds_bytes_ck(a.bits, a.group, R, tv, CK) > lds_cap || (a.kind == kQlStream && a.tm != 1 && a.tm != 2) ||
        (gemm && (a.tm != kQlGemmTm || TN != kQlGemmTn || a.splits != ql_gemm_splits(a.T, a.n))))
      return violation("staged product geometry (kc %lld, ld %lld)", a.kc, a.codes_ld), hipErrorInvalidValue;
    if (gemm) {
      // paired activation units: the two natural pieces and the two stored
      // operands of each unit lie inside the chunk, and the stored operands
      // of all units tile the chunk exactly once
      const bool bf = a.xt == BRQ_BF16;
      const int NC2 = a.group / 4, UT = CK / 16;
      std::vector<int> seen(CK / 8, 0);
      for (int u = 0; u < UT; ++u) {
        const int n0 = ql_gemm_nat0(u, NC2, bf), n1 = ql_gemm_nat1(u, NC2, bf), o0 = ql_gemm_op0(u, NC2);
        if (n0 < 0 || n1 + 8 > CK || o0 + 16 > CK || n0 % 8 || n1 % 8 || o0 % 8)
          return violation("activation unit %lld at %lld", u, n0), hipErrorInvalidValue;
        ++seen[o0 / 8];
        ++seen[o0 / 8 + 1];
      }
      for (int q = 0; q < CK / 8; ++q)
        if (seen[q] != 1) return violation("activation operand slot %lld stored %lld times", q, seen[q]), hipErrorInvalidValue;
      if (ql_gemm_lds_bytes(a.bits, a.group, kQlTok * kQlGemmTm) > 160 * 1024)
        return violation("gemm LDS %lld bytes", (int64_t)ql_gemm_lds_bytes(a.bits, a.group, kQlTok * kQlGemmTm), 0),
               hipErrorInvalidValue;
    }
    {
      // staged pieces per thread divide exactly; activation reads stay inside a token's chunk row
      const int NG = CK / a.group;
      const int NT = gemm ? kQlGemmThreads : kQlThreads;
      if ((R * (CB / 16)) % NT || (R * NG) % NT || (kQlTok * a.tm * (CK / 8)) % NT)
        return violation("staging pieces (rows %lld)", R, 0), hipErrorInvalidValue;
      const bool bf = a.xt == BRQ_BF16;
      for (int gi = 0; gi < NG; ++gi)
        for (int lg = 0; lg < 4; ++lg)
          for (int sp = 0; sp < NC / 16; ++sp) {
            const int64_t lo = gi * a.group + lg * NC + (bf ? 16 * sp : 8 * sp);
            const int64_t hi = lo + (bf ? 8 : NC / 2) + 8;
            if (lo < 0 || 2 * hi > 2 * CK || (2 * lo) % 16)
              return violation("LDS activation read at %lld (group %lld)", 2 * lo, gi), hipErrorInvalidValue;
          }
      const int XP = ql_xpitch(CK);
      if ((int64_t)tv * XP % 16 || XP < 2 * CK)
        return violation("LDS activation pitch %lld", XP, 0), hipErrorInvalidValue;
    }
    if (PB % 16 || ((int64_t)R * PB) % 16) return violation("LDS code pitch %lld", PB, 0), hipErrorInvalidValue;
    for (int r = 0; r < R; ++r)
      for (int gi = 0; gi < CK / a.group; ++gi)
        for (int lg = 0; lg < 4; ++lg) {
          const int off = r * PB + gi * (a.group * a.bits / 8) + lg * NB;
          if (off + NB > r * PB + CB || off % (NB % 4 == 0 ? 4 : 2))
            return violation("LDS code word at %lld (row %lld)", off, r), hipErrorInvalidValue;
        }
  }
  std::vector<uint8_t> cover((size_t)(a.splits * a.T * a.m), 0);
  for (int64_t bid = 0; bid < nb; ++bid) {
    const QlTile t = ql_tile(a, bid);
    if (t.ct >= ql_ctiles(a) || t.tt >= ql_ttiles(a) || t.split >= a.splits)
      return violation("quantized linear block %lld", bid, 0), hipErrorInvalidValue;
    const int64_t kb = t.split * a.kc, ke = std::min(kb + a.kc, a.n);
    for (int w = 0; w < 4; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const int lr = lane & 15, lg = lane >> 4;
        const int64_t ob = t.ct * ((int64_t)kQlOut * TN) + (int64_t)16 * TN * w + lr;
        for (int tn = 0; tn < TN; ++tn)
          if (ob + 16 * tn >= a.m) return violation("weight row %lld", ob + 16 * tn, 0), hipErrorInvalidValue;
        for (int64_t g0 = kb; g0 < ke; g0 += a.group) {
          if (g0 / a.group >= a.scales_ld) return violation("scale column %lld", g0 / a.group, 0), hipErrorInvalidValue;
          // the lane's code chunks: NB bytes, 4-byte words when NB % 4 == 0, else 16-bit pieces
          for (int tn = 0; tn < TN; ++tn) {
            const int64_t off = ql_code_off(a, ob + 16 * tn, g0 + (int64_t)lg * NC);
            if (off < 0 || off + NB > a.m * a.codes_ld || off % (NB % 4 == 0 ? 4 : 2))
              return violation("code chunk at %lld", off, 0), hipErrorInvalidValue;
          }
          for (int st = 0; st < NC / 8; ++st) {
            const int64_t k = g0 + (int64_t)lg * NC + 8 * st;
            if (k + 8 > ke) return violation("input columns %lld", k, 0), hipErrorInvalidValue;
            for (int tm = 0; tm < a.tm; ++tm) {
              const int64_t tok = (t.tt * a.tm + tm) * kQlTok + lr;
              if (tok < a.T && (tok * a.ldx + k) % 8) return violation("activation vector at %lld", tok * a.ldx + k, 0), hipErrorInvalidValue;
            }
          }
        }
        for (int tm = 0; tm < a.tm; ++tm)
          for (int i = 0; i < 4; ++i) {
            const int64_t tk = (t.tt * a.tm + tm) * kQlTok + 4 * lg + i;
            for (int tn = 0; tn < TN; ++tn)
              if (tk < a.T && cover[(size_t)((t.split * a.T + tk) * a.m + ob + 16 * tn)]++)
                return violation("partial (%lld, %lld) written twice", tk, ob + 16 * tn), hipErrorInvalidValue;
          }
      }
  }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return violation("partial %lld written %lld times", (int64_t)i, cover[i]), hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_ql_reduce(const float*, int splits, int64_t T, int64_t m, void*, int ot,
                            int64_t ldo, hipStream_t) {
  ++g_launches;
  if (splits < 1 || T < 1 || m < 1 || ldo < m || (ot != BRQ_F32 && ot != BRQ_F16 && ot != BRQ_BF16))
    return violation("reduce geometry (splits %lld, ld %lld)", splits, ldo), hipErrorInvalidValue;
  return hipSuccess;
}

// ---------------------------------------------------------------- ORP GEO

static hipError_t walk_orp(const OrpArgs& a, bool quant) {
  ++g_launches;
  const int bits = a.bits, g = a.group, S = a.stride;
  if (bits < 2 || bits > 5 || g % kOrpPerLane || g > kOrpChunk || (g & (g - 1)) || S < 1 ||
      (S & (S - 1)) || 2 * S > g || a.n % g)
    return violation("ORP geometry (group %lld, stride %lld)", g, S), hipErrorInvalidValue;
  if (a.chunks != (a.n + kOrpChunk - 1) / kOrpChunk)
    return violation("ORP chunks per row %lld for n %lld", a.chunks, a.n), hipErrorInvalidValue;
  if ((1 << a.lg_group) != g || (1 << a.lg_stride) != S || a.codes_ld != a.n * bits / 8 ||
      a.signs_ld != a.n / 16 || a.coef_ld != 2 * (a.n / g) || a.n >= ((int64_t)1 << 31))
    return violation("ORP strides (log2 group %lld, log2 stride %lld)", a.lg_group, a.lg_stride), hipErrorInvalidValue;
  for (int64_t i = 0; i < 4 * S + 64; ++i)  // the shift form of the pair number
    if (orp_pair(i, S) % (2 * S) < S && (int64_t)orp_pair_lg((uint32_t)i, a.lg_stride) != orp_pair(i, S))
      return violation("ORP pair number of %lld", i, S), hipErrorInvalidValue;
  const int lpg = g / kOrpPerLane;
  const int64_t cb = a.n * bits / 8, sb = a.n / 16, ng = a.n / g;
  std::vector<uint8_t> code_cov((size_t)(a.m * cb), 0), sign_cov((size_t)(a.m * sb), 0);
  std::vector<uint8_t> coef_cov((size_t)(a.m * ng), 0), elem_cov((size_t)(a.m * a.n), 0);
  const int64_t waves = orp_waves(a), total = orp_total_chunks(a);
  if (orp_blocks(a) * (kOrpThreads / 64) < waves || waves * kOrpChunksPerWave < total)
    return violation("ORP grid of %lld blocks for %lld chunks", orp_blocks(a), total), hipErrorInvalidValue;
  for (int64_t wv = 0; wv < waves; ++wv)
  for (int jc = 0; jc < kOrpChunksPerWave; ++jc) {
    const int64_t ci = wv * kOrpChunksPerWave + jc;
    if (ci >= total) break;
    int64_t row, c0;
    orp_chunk(a, ci, &row, &c0);
    if (row < 0 || row >= a.m || c0 % g) return violation("ORP chunk %lld at row %lld", ci, row), hipErrorInvalidValue;
    for (int lane = 0; lane < 64; ++lane) {
      const int64_t col = c0 + kOrpPerLane * lane;
      const bool valid = col < a.n;
      // a group's lanes are all valid or all not
      const int lead = lane & ~(lpg - 1);
      if (valid != (c0 + kOrpPerLane * lead < a.n))
        return violation("ORP group straddles the row end at column %lld (n %lld)", col, a.n), hipErrorInvalidValue;
      if (S >= kOrpPerLane) {
        const int xm = S / kOrpPerLane, partner = lane ^ xm;
        if ((partner & ~(lpg - 1)) != lead)
          return violation("ORP pair partner lane %lld outside the group of lane %lld", partner, lane), hipErrorInvalidValue;
        if (valid && ((lane & (lpg - 1)) & xm) == 0 && (col + S) / (2 * S) != col / (2 * S))
          return violation("ORP pair at column %lld leaves its micro-block", col, S), hipErrorInvalidValue;
      }
      if (!valid) continue;
      if (col + kOrpPerLane > a.n) return violation("ORP lane reads past the row (%lld, n %lld)", col, a.n), hipErrorInvalidValue;
      for (int j = 0; j < kOrpPerLane; ++j) elem_cov[(size_t)(row * a.n + col + j)]++;
      // codes
      const int64_t cbyte = col * bits / 8;
      for (int b = 0; b < bits; ++b) {
        if (cbyte + b >= cb) return violation("ORP code byte %lld of a %lld-byte row", cbyte + b, cb), hipErrorInvalidValue;
        if (quant) code_cov[(size_t)(row * cb + cbyte + b)]++;
      }
      // sign bytes
      if (S < kOrpPerLane) {
        if (col / 16 >= sb) return violation("ORP sign byte %lld of %lld", col / 16, sb), hipErrorInvalidValue;
        if (quant && (lane & 1) == 0) sign_cov[(size_t)(row * sb + col / 16)]++;
      } else {
        const bool first = ((lane & (lpg - 1)) & (S / kOrpPerLane)) == 0;
        const int64_t fc = first ? col : col - S;
        const int64_t byte = orp_pair(fc, S) / 8;
        if (fc < 0 || orp_pair(fc, S) % 8 || byte >= sb)
          return violation("ORP sign byte %lld for column %lld", byte, col), hipErrorInvalidValue;
        if (quant && first) sign_cov[(size_t)(row * sb + byte)]++;
      }
      // coefficients
      const int64_t ci = row * ng + col / g;
      if (2 * ci + 1 >= 2 * a.m * ng) return violation("ORP coefficient %lld of %lld", ci, a.m * ng), hipErrorInvalidValue;
      if (quant && (lane & (lpg - 1)) == 0) coef_cov[(size_t)ci]++;
      // input / output rows
      const int64_t ld = quant ? a.ldw : a.ldo;
      if (ld < a.n || row * ld + col + kOrpPerLane > a.m * ld)
        return violation("ORP element %lld outside %lld", row * ld + col, a.m * ld), hipErrorInvalidValue;
    }
  }
  for (size_t i = 0; i < elem_cov.size(); ++i)
    if (elem_cov[i] != 1) return violation("ORP element %lld handled %lld times", (int64_t)i, elem_cov[i]), hipErrorInvalidValue;
  if (quant) {
    for (size_t i = 0; i < code_cov.size(); ++i)
      if (code_cov[i] != 1) return violation("ORP code byte %lld written %lld times", (int64_t)i, code_cov[i]), hipErrorInvalidValue;
    for (size_t i = 0; i < sign_cov.size(); ++i)
      if (sign_cov[i] != 1) return violation("ORP sign byte %lld written %lld times", (int64_t)i, sign_cov[i]), hipErrorInvalidValue;
    for (size_t i = 0; i < coef_cov.size(); ++i)
      if (coef_cov[i] != 1) return violation("ORP coefficients %lld written %lld times", (int64_t)i, coef_cov[i]), hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_orp_quant(const OrpArgs& a, hipStream_t) { return walk_orp(a, true); }
hipError_t launch_orp_dequant(const OrpArgs& a, hipStream_t) { return walk_orp(a, false); }

}  // namespace brq
