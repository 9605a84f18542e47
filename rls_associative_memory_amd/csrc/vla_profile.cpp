// Opt-in per-kernel timing with HIP events (see vla_profile_* in vla.h).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "vla.h"
#include "vla_internal.h"

namespace vla {
namespace {

struct Pending {
  const char *name;
  hipEvent_t ev0, ev1;
};
struct Total {
  std::string name;
  double ms = 0.0;
  int64_t launches = 0;
};

std::atomic<bool> g_on{false};
thread_local bool t_quiet = false;
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::vector<Total> g_totals;

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

// Wait for every pending pair and fold it into the totals (caller holds g_mu).
void resolve_locked() {
  for (const Pending &p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.ev1) == hipSuccess && hipEventElapsedTime(&ms, p.ev0, p.ev1) == hipSuccess) {
      Total *t = nullptr;
      for (Total &x : g_totals)
        if (x.name == p.name) t = &x;
      if (t == nullptr) {
        g_totals.push_back(Total{p.name, 0.0, 0});
        t = &g_totals.back();
      }
      t->ms += ms;
      t->launches += 1;
    }
    g_free.push_back(p.ev0);
    g_free.push_back(p.ev1);
  }
  g_pending.clear();
}

}  // namespace

ProfQuiet::ProfQuiet() : prev_(t_quiet) { t_quiet = true; }
ProfQuiet::~ProfQuiet() { t_quiet = prev_; }

ProfScope::ProfScope(const char *name, hipStream_t s) : name_(name), stream_(s) {
  if (t_quiet || !g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  ev0_ = take_event();
  ev1_ = take_event();
  if (ev0_ != nullptr && ev1_ != nullptr) {
    active_ = hipEventRecord(ev0_, stream_) == hipSuccess;
  }
}

ProfScope::~ProfScope() {
  if (!active_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(ev1_, stream_) == hipSuccess) {
    g_pending.push_back(Pending{name_, ev0_, ev1_});
  } else {
    g_free.push_back(ev0_);
    g_free.push_back(ev1_);
  }
}

}  // namespace vla

extern "C" {

vla_status_t vla_profile_enable(int32_t enable) {
  vla::g_on.store(enable != 0);
  return VLA_SUCCESS;
}

vla_status_t vla_profile_reset(void) {
  std::lock_guard<std::mutex> lk(vla::g_mu);
  vla::resolve_locked();
  vla::g_totals.clear();
  return VLA_SUCCESS;
}

int32_t vla_profile_count(void) {
  std::lock_guard<std::mutex> lk(vla::g_mu);
  vla::resolve_locked();
  return static_cast<int32_t>(vla::g_totals.size());
}

vla_status_t vla_profile_get(int32_t index, char *name, size_t name_cap, double *total_ms,
                             int64_t *launches) {
  std::lock_guard<std::mutex> lk(vla::g_mu);
  vla::resolve_locked();
  if (index < 0 || index >= static_cast<int32_t>(vla::g_totals.size())) return VLA_ERROR_INVALID_VALUE;
  const vla::Total &t = vla::g_totals[index];
  if (name != nullptr && name_cap > 0) {
    std::strncpy(name, t.name.c_str(), name_cap - 1);
    name[name_cap - 1] = '\0';
  }
  if (total_ms != nullptr) *total_ms = t.ms;
  if (launches != nullptr) *launches = t.launches;
  return VLA_SUCCESS;
}

}  // extern "C"
