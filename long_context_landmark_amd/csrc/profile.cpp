// Opt-in per-kernel timing with HIP events on the launching stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hils.h"
#include "hils_launch.h"

namespace hils {
namespace prof {
namespace {
struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Acc {
  std::string name;
  double ms;
  long calls;
};
std::mutex g_mu;
std::atomic<bool> g_on{false};  // read by every launch without the lock
std::vector<Pending> g_pending;
std::vector<Acc> g_acc;
}  // namespace

bool make(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_on.load(std::memory_order_relaxed)) return false;
  if (hipEventCreate(start) != hipSuccess) return false;
  if (hipEventCreate(stop) != hipSuccess) {
    (void)hipEventDestroy(*start);
    return false;
  }
  return true;
}

void add(const char* name, hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({name, start, stop});
}

void collect() {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) ms = 0.f;
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
    bool found = false;
    for (auto& a : g_acc)
      if (a.name == p.name) {
        a.ms += ms;
        a.calls += 1;
        found = true;
        break;
      }
    if (!found) g_acc.push_back({p.name, (double)ms, 1});
  }
  g_pending.clear();
}
}  // namespace prof
}  // namespace hils

extern "C" {

void hils_profile_enable(int on) {
  hils::prof::collect();
  std::lock_guard<std::mutex> lk(hils::prof::g_mu);
  hils::prof::g_on.store(on != 0);
  hils::prof::g_acc.clear();
}

int hils_profile_read(char* names, int name_stride, double* total_ms, long* calls, int max_kernels) {
  hils::prof::collect();
  std::lock_guard<std::mutex> lk(hils::prof::g_mu);
  int n = 0;
  for (auto& a : hils::prof::g_acc) {
    if (n >= max_kernels) break;
    if (names && name_stride > 0) {
      std::strncpy(names + (size_t)n * name_stride, a.name.c_str(), (size_t)name_stride - 1);
      names[(size_t)n * name_stride + name_stride - 1] = 0;
    }
    if (total_ms) total_ms[n] = a.ms;
    if (calls) calls[n] = a.calls;
    ++n;
  }
  return (int)hils::prof::g_acc.size();
}
}
