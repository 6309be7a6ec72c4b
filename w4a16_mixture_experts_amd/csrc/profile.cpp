// Optional per-kernel timing for benchmarks: when enabled, every kernel of the library is
// launched with a hipEvent pair that stamps the kernel's own start and end on its launch
// stream (hipExtLaunchKernelGGL); exmoe_profile_read synchronizes those events and returns
// per-kernel totals. Off by default; never active while a stream is being captured.
#include <hip/hip_runtime.h>

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

}  // extern "C"
