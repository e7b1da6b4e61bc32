// Per-launch timing registry behind favor_timing_enable / favor_timing_read.
#include "../../include/favor.h"
#include "favor_timing.hpp"

#include <mutex>
#include <string>
#include <vector>

namespace favor {
namespace {
struct Rec {
  const char* name;
  hipEvent_t a = nullptr, b = nullptr;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;

void clear_locked() {
  for (auto& r : g_recs) {
    if (r.a) hipEventDestroy(r.a);
    if (r.b) hipEventDestroy(r.b);
  }
  g_recs.clear();
}
}  // namespace

bool timing_on() { return g_on; }

bool timing_pair(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return false;
  Rec r;
  r.name = name;
  if (hipEventCreate(&r.a) != hipSuccess) return false;
  if (hipEventCreate(&r.b) != hipSuccess) {
    hipEventDestroy(r.a);
    return false;
  }
  g_recs.push_back(r);
  *start = r.a;
  *stop = r.b;
  return true;
}
}  // namespace favor

extern "C" {

favor_status favor_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(favor::g_mu);
  favor::clear_locked();
  favor::g_on = on != 0;
  return FAVOR_OK;
}

int favor_timing_read(const char** names, float* ms, int cap) {
  std::lock_guard<std::mutex> lk(favor::g_mu);
  const int n = (int)favor::g_recs.size();
  for (int i = 0; i < n && i < cap; ++i) {
    auto& r = favor::g_recs[i];
    float t = -1.f;
    if (hipEventSynchronize(r.b) == hipSuccess) hipEventElapsedTime(&t, r.a, r.b);
    if (names) names[i] = r.name;
    if (ms) ms[i] = t;
  }
  return n;
}

}  // extern "C"
