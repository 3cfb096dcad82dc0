// Thin HIP runtime wrappers used by the host layer.
#include <cstdio>

#include "brq_internal.h"

namespace brq {

hipError_t rt_get_device(int* dev) { return hipGetDevice(dev); }

hipError_t rt_malloc(void** p, size_t bytes) { return hipMalloc(p, bytes); }

hipError_t rt_copy_to_device(void* dst, const void* src, size_t bytes) {
  return hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
}

hipError_t rt_copy_to_host(void* dst, const void* src, size_t bytes) {
  return hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
}

hipError_t rt_cu_count(int dev, int* cus) {
  return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
}

void rt_free(void* p) {
  if (p) (void)hipFree(p);
}

}  // namespace brq

// ---------------------------------------------------------------- kernel timing

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

namespace brq {
namespace {

struct Pending {
  int name;
  hipEvent_t a, b;
};

struct Totals {
  std::string name;
  double ms = 0;
  int64_t launches = 0;
};

std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<Pending> g_pending;
std::vector<Totals> g_totals;

int name_index(const char* name) {
  for (size_t i = 0; i < g_totals.size(); ++i)
    if (g_totals[i].name == name) return (int)i;
  g_totals.push_back(Totals{name, 0.0, 0});
  return (int)g_totals.size() - 1;
}

hipError_t drain() {
  for (Pending& p : g_pending) {
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, p.a, p.b);
    if (e != hipSuccess) return e;
    g_totals[p.name].ms += ms;
    g_totals[p.name].launches += 1;
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  g_pending.clear();
  return hipSuccess;
}

}  // namespace

int prof_begin(const char* name, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  Pending p;
  p.name = name_index(name);
  if (hipEventCreate(&p.a) != hipSuccess) return -1;
  if (hipEventCreate(&p.b) != hipSuccess) {
    (void)hipEventDestroy(p.a);
    return -1;
  }
  if (hipEventRecord(p.a, s) != hipSuccess) {
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
    return -1;
  }
  g_pending.push_back(p);
  return (int)g_pending.size() - 1;
}

void prof_end(int token, hipStream_t s) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (token < (int)g_pending.size()) (void)hipEventRecord(g_pending[token].b, s);
}

}  // namespace brq

extern "C" {

brq_status brq_profile_enable(int32_t on) {
  brq::g_prof_on.store(on != 0);
  return BRQ_OK;
}

brq_status brq_profile_reset(void) {
  std::lock_guard<std::mutex> lk(brq::g_prof_mu);
  if (brq::drain() != hipSuccess) return BRQ_ERR_HIP;
  brq::g_totals.clear();
  return BRQ_OK;
}

int32_t brq_profile_count(void) {
  std::lock_guard<std::mutex> lk(brq::g_prof_mu);
  return (int32_t)brq::g_totals.size();
}

brq_status brq_profile_read(int32_t idx, char* name, size_t name_len, double* total_ms,
                            int64_t* launches) {
  std::lock_guard<std::mutex> lk(brq::g_prof_mu);
  if (brq::drain() != hipSuccess) return BRQ_ERR_HIP;
  if (idx < 0 || idx >= (int32_t)brq::g_totals.size() || !name || !name_len || !total_ms ||
      !launches)
    return BRQ_ERR_INVALID_ARGUMENT;
  const brq::Totals& t = brq::g_totals[idx];
  snprintf(name, name_len, "%s", t.name.c_str());
  *total_ms = t.ms;
  *launches = t.launches;
  return BRQ_OK;
}

}  // extern "C"
