// Per-kernel timing with HIP events.  Off by default; while on, every kernel
// launch of the library is bracketed by two events recorded on the launch's
// own stream, and moe_profile_collect() turns the pairs into per-kernel
// totals.  Events come from a pool, so steady-state recording allocates
// nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "launch.h"

namespace moe {
namespace {

struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Stat {
  std::string name;
  double ms = 0.0;
  long long launches = 0;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::vector<Stat> g_stats;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Pending p{name, take_event(), take_event()};
  if (!p.a || !p.b) return;
  if (hipEventRecord(p.a, s) != hipSuccess) return;
  g_pending.push_back(p);
  slot = (int)g_pending.size() - 1;
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (slot < (int)g_pending.size()) hipEventRecord(g_pending[slot].b, stream);
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (on) {
    g_stats.clear();
    for (auto& p : g_pending) {
      g_pool.push_back(p.a);
      g_pool.push_back(p.b);
    }
    g_pending.clear();
  }
  g_on.store(on ? 1 : 0);
  return MOE_OK;
}

int moe_profile_collect(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      Stat* st = nullptr;
      for (auto& s : g_stats)
        if (s.name == p.name) st = &s;
      if (!st) {
        g_stats.push_back(Stat{p.name, 0.0, 0});
        st = &g_stats.back();
      }
      st->ms += ms;
      st->launches += 1;
    }
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
  return (int)g_stats.size();
}

moe_status moe_profile_entry(int i, char* name, size_t name_len, double* total_ms,
                             long long* launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int)g_stats.size() || !name || name_len == 0 || !total_ms || !launches)
    return MOE_ERR_INVALID_ARG;
  std::strncpy(name, g_stats[i].name.c_str(), name_len - 1);
  name[name_len - 1] = 0;
  *total_ms = g_stats[i].ms;
  *launches = g_stats[i].launches;
  return MOE_OK;
}

}  // extern "C"
