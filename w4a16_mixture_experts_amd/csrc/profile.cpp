// Optional per-kernel timing for benchmarks. Events: when enabled, every kernel of the
// library is launched with a hipEvent pair on its launch stream (hipExtLaunchKernelGGL);
// exmoe_profile_read synchronizes those events and returns per-kernel totals (never active
// while a stream is being captured). Spans: when enabled, each launch of the expert-layer
// kernels takes a device slot in which its workgroups stamp the GPU clock at start and end
// (also inside a captured graph); exmoe_span_read sums max(end) - min(start) per kernel.
// Both are off by default.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "exmoe.h"

namespace exmoe {

namespace {
struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Totals {
  double ms = 0.0;
  uint64_t n = 0;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::map<std::string, Totals> g_totals;
// launch span slots: [cap][kSpanSub][2] u64 on the device (min start, max end), one per launch
unsigned long long* g_span = nullptr;
int g_span_cap = 0;
std::vector<const char*> g_span_names;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;
  return st != hipStreamCaptureStatusNone;
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || capturing(s)) return;
  a_ = take_event();
  b_ = take_event();
  if (!a_ || !b_) {
    if (a_) g_free.push_back(a_);
    if (b_) g_free.push_back(b_);
    a_ = b_ = nullptr;
  }
}

unsigned long long* ProfScope::span() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_span || (int)g_span_names.size() >= g_span_cap) return nullptr;
  g_span_names.push_back(name_);
  return g_span + 2 * kSpanSub * (g_span_names.size() - 1);
}

ProfScope::~ProfScope() {
  if (!a_ || !b_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (used_) {
    g_pending.push_back({name_, a_, b_});
  } else {
    g_free.push_back(a_);
    g_free.push_back(b_);
  }
}

}  // namespace exmoe

using namespace exmoe;

extern "C" {

int exmoe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return EXMOE_OK;
}

int exmoe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    (void)hipEventSynchronize(p.b);
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.clear();
  g_totals.clear();
  return EXMOE_OK;
}

int exmoe_profile_read(const char* kernel, double* total_ms, uint64_t* launches) {
  if (!kernel || !total_ms || !launches) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "NULL argument");
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return hip_error(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, p.a, p.b);
    if (e != hipSuccess) return hip_error(e, "hipEventElapsedTime");
    Totals& t = g_totals[p.name];
    t.ms += ms;
    t.n += 1;
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.clear();
  auto it = g_totals.find(kernel);
  *total_ms = it == g_totals.end() ? 0.0 : it->second.ms;
  *launches = it == g_totals.end() ? 0 : it->second.n;
  return EXMOE_OK;
}

int exmoe_span_enable(int max_launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_span) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_error(e, "hipDeviceSynchronize");
    (void)hipFree(g_span);
  }
  g_span = nullptr;
  g_span_cap = 0;
  g_span_names.clear();
  if (max_launches < 0) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "max_launches must be >= 0");
  if (max_launches == 0) return EXMOE_OK;
  hipError_t e = hipMalloc(&g_span, sizeof(unsigned long long) * 2 * kSpanSub * (size_t)max_launches);
  if (e != hipSuccess) {
    g_span = nullptr;
    return hip_error(e, "hipMalloc");
  }
  g_span_cap = max_launches;
  e = span_fill(g_span, max_launches * kSpanSub, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return e == hipSuccess ? EXMOE_OK : hip_error(e, "span fill");
}

int exmoe_span_clear(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_span) return EXMOE_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = span_fill(g_span, g_span_cap * kSpanSub, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return e == hipSuccess ? EXMOE_OK : hip_error(e, "span fill");
}

int exmoe_span_read(const char* kernel, double* total_us, uint64_t* launches) {
  if (!kernel || !total_us || !launches) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "NULL argument");
  std::lock_guard<std::mutex> lk(g_mu);
  *total_us = 0.0;
  *launches = 0;
  const size_t n = g_span_names.size();
  if (!g_span || n == 0) return EXMOE_OK;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return hip_error(e, "wall clock rate");
  if (khz <= 0) return set_error(EXMOE_ERR_UNSUPPORTED, "wall clock rate unknown");
  std::vector<unsigned long long> h(2 * kSpanSub * n);
  e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h.data(), g_span, sizeof(unsigned long long) * h.size(), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_error(e, "span copy");
  for (size_t i = 0; i < n; i++) {
    if (std::strcmp(g_span_names[i], kernel) != 0) continue;
    unsigned long long a = ~0ull, b = 0;
    for (int q = 0; q < kSpanSub; q++) {
      a = std::min(a, h[2 * (kSpanSub * i + q)]);
      b = std::max(b, h[2 * (kSpanSub * i + q) + 1]);
    }
    if (a == ~0ull || b < a) continue;   // slot not run since the last clear
    *total_us += (double)(b - a) * 1000.0 / (double)khz;
    *launches += 1;
  }
  return EXMOE_OK;
}

}  // extern "C"
