// Kernel-level timing log (diagnostics).  When enabled, each library call
// brackets its dominant kernel with a pair of HIP events recorded on the call's
// own stream; qn_trace_read() waits for them and returns the durations.

#include <atomic>
#include <mutex>
#include <vector>

#include "qn_internal.h"

namespace qn {
namespace {

struct Entry {
  int kind;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Entry> g_log;
std::vector<hipEvent_t> g_pool;

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

TraceScope::TraceScope(int kind, hipStream_t s) : kind_(kind), stream_(s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  stop_ = take_event();
  if (start_ && stop_ && hipEventRecord(start_, s) == hipSuccess) return;
  if (start_) g_pool.push_back(start_);
  if (stop_) g_pool.push_back(stop_);
  start_ = stop_ = nullptr;
}

TraceScope::~TraceScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    g_log.push_back(Entry{kind_, start_, stop_});
  } else {
    g_pool.push_back(start_);
    g_pool.push_back(stop_);
  }
}

}  // namespace qn

extern "C" {

int qn_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(qn::g_mu);
  for (auto &e : qn::g_log) {
    qn::g_pool.push_back(e.start);
    qn::g_pool.push_back(e.stop);
  }
  qn::g_log.clear();
  qn::g_on.store(on != 0);
  return QN_OK;
}

int qn_trace_read(int *kinds, float *ms, int cap) {
  if (cap < 0 || (cap > 0 && (!kinds || !ms))) return -QN_ERR_NULL;
  std::lock_guard<std::mutex> lk(qn::g_mu);
  int n = 0;
  int status = 0;
  for (auto &e : qn::g_log) {
    if (n < cap) {
      float t = -1.0f;
      if (hipEventSynchronize(e.stop) != hipSuccess || hipEventElapsedTime(&t, e.start, e.stop) != hipSuccess)
        status = -QN_ERR_HIP;
      kinds[n] = e.kind;
      ms[n] = t;
      ++n;
    }
    qn::g_pool.push_back(e.start);
    qn::g_pool.push_back(e.stop);
  }
  qn::g_log.clear();
  return status ? status : n;
}

}  // extern "C"
