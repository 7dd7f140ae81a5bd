// Optional per-stage timing (diagnostics): when enabled, the library brackets
// the launches of each timed stage with a pair of HIP events on the caller's
// stream, and gptq_timing_read() sums their elapsed times.  Off by default;
// when off, a scope costs one atomic load.
#include <atomic>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace gq {
namespace {

std::atomic<int> g_enabled{0};
std::mutex g_mu;
struct Pair { int which; hipEvent_t a, b; };
std::vector<Pair> g_pairs;           // recorded since the last read
std::vector<hipEvent_t> g_free;      // event pool

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

}  // namespace

TimerScope::TimerScope(int which, hipStream_t s) : which_(which), s_(s) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = take_event();
  if (a_ && hipEventRecord(a_, s) != hipSuccess) {
    g_free.push_back(a_);
    a_ = nullptr;
  }
}

TimerScope::~TimerScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (b && hipEventRecord(b, s_) == hipSuccess) {
    g_pairs.push_back({which_, a_, b});
  } else {
    g_free.push_back(a_);
    if (b) g_free.push_back(b);
  }
}

int timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pairs) {
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pairs.clear();
  g_enabled.store(on ? 1 : 0);
  return 0;
}

hipError_t timing_read(float* ms, int n) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (int i = 0; i < n; ++i) ms[i] = 0.f;
  hipError_t err = hipSuccess;
  for (auto& p : g_pairs) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(p.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, p.a, p.b);
    if (e != hipSuccess) err = e;
    else if (p.which >= 0 && p.which < n) ms[p.which] += t;
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pairs.clear();
  return err;
}

}  // namespace gq
