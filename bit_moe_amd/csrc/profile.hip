// Optional per-kernel launch timing (off unless bitmoe_profile_start() was
// called): every launch gets a start/stop event pair that hipExtLaunchKernel
// stamps with the kernel's own execution start and end.
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "bitmoe.h"
#include "internal.h"

namespace bm {
namespace {

struct Rec {
  const char *name;
  hipEvent_t a, b;
};

struct Agg {
  std::string name;
  double ms = 0.0;
  int64_t launches = 0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
std::vector<Agg> g_aggs;

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

void prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r{name, take_event(), take_event()};
  if (!r.a || !r.b) return;
  g_recs.push_back(r);
  *start = r.a;
  *stop = r.b;
}

}  // namespace bm

extern "C" {

int bitmoe_profile_start(void) {
  std::lock_guard<std::mutex> lk(bm::g_mu);
  for (auto &r : bm::g_recs) {
    bm::g_pool.push_back(r.a);
    bm::g_pool.push_back(r.b);
  }
  bm::g_recs.clear();
  bm::g_aggs.clear();
  bm::g_on = true;
  return BITMOE_OK;
}

int bitmoe_profile_stop(void) {
  std::lock_guard<std::mutex> lk(bm::g_mu);
  bm::g_on = false;
  for (auto &r : bm::g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return BITMOE_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return BITMOE_EHIP;
    bm::Agg *agg = nullptr;
    for (auto &g : bm::g_aggs)
      if (g.name == r.name) agg = &g;
    if (!agg) {
      bm::g_aggs.push_back(bm::Agg{r.name});
      agg = &bm::g_aggs.back();
    }
    agg->ms += ms;
    agg->launches += 1;
  }
  return int(bm::g_aggs.size());
}

int bitmoe_profile_get(int32_t i, const char **name, double *total_ms, int64_t *launches) {
  std::lock_guard<std::mutex> lk(bm::g_mu);
  if (i < 0 || i >= int(bm::g_aggs.size()) || !name || !total_ms || !launches) return BITMOE_EINVAL;
  *name = bm::g_aggs[i].name.c_str();
  *total_ms = bm::g_aggs[i].ms;
  *launches = bm::g_aggs[i].launches;
  return BITMOE_OK;
}

}  // extern "C"
