// Per-kernel timing for benchmarks: hipEvent pairs recorded on each kernel's
// launch stream while enabled, aggregated by kernel name on request.
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "rz.h"
#include "rz_internal.h"

namespace rz {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_open;   // start events waiting for their stop, per record slot
std::vector<std::string> g_names;
std::vector<double> g_ms;
std::vector<int64_t> g_n;

void clear_locked() {
  for (auto& r : g_recs) {
    if (r.a) (void)hipEventDestroy(r.a);
    if (r.b) (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
  g_names.clear();
  g_ms.clear();
  g_n.clear();
}

}  // namespace

bool profile_enabled() { return g_on.load(std::memory_order_relaxed); }

void profile_record(const char* name, hipStream_t s, bool start) {
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return;
  (void)hipEventRecord(e, s);
  if (start) {
    g_recs.push_back(Rec{name, e, nullptr});
  } else {
    // close the most recent open record of this name
    for (auto it = g_recs.rbegin(); it != g_recs.rend(); ++it)
      if (it->name == name && it->b == nullptr) {
        it->b = e;
        return;
      }
    (void)hipEventDestroy(e);
  }
}

}  // namespace rz

extern "C" {

int rz_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(rz::g_mu);
  rz::clear_locked();
  rz::g_on.store(on != 0);
  return RZ_OK;
}

int rz_profile_count(void) {
  std::lock_guard<std::mutex> lk(rz::g_mu);
  std::map<std::string, std::pair<double, int64_t>> agg;
  for (auto& r : rz::g_recs) {
    if (!r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return -RZ_EHIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return -RZ_EHIP;
    auto& v = agg[r.name];
    v.first += ms;
    v.second += 1;
  }
  rz::g_names.clear();
  rz::g_ms.clear();
  rz::g_n.clear();
  for (auto& kv : agg) {
    rz::g_names.push_back(kv.first);
    rz::g_ms.push_back(kv.second.first);
    rz::g_n.push_back(kv.second.second);
  }
  return int(rz::g_names.size());
}

int rz_profile_get(int i, const char** name, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(rz::g_mu);
  if (i < 0 || i >= int(rz::g_names.size()) || !name || !total_ms || !launches) return RZ_EINVAL;
  *name = rz::g_names[i].c_str();
  *total_ms = rz::g_ms[i];
  *launches = rz::g_n[i];
  return RZ_OK;
}

}  // extern "C"
