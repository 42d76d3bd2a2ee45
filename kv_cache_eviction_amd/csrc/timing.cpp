// Opt-in per-launch kernel timing: when enabled, every kernel the library
// launches is bracketed by a pair of HIP events recorded on the launch stream.
// Reading a record synchronises on its stop event.  Meant for benchmarks and
// profiling; off by default, and then costs one relaxed atomic load per launch.
#include "timing.hpp"

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

namespace kvs {
namespace {

struct Record {
  const char *name;
  hipEvent_t start, stop;
};

std::atomic<int> g_enabled{0};
std::mutex g_mu;
std::vector<Record> g_records;  // recorded launches since the last reset
std::vector<hipEvent_t> g_pool;  // events free for reuse

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // timing-only events: without the system-scope fence a default event
  // performs when it is recorded (an L2 write-back and invalidation), so the
  // bracket measures the kernel and does not slow the work that follows it
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

TimedLaunch::TimedLaunch(const char *name, hipStream_t st) : stream_(st), index_(-1) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Record r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  hipEventRecord(r.start, st);
  g_records.push_back(r);
  index_ = (int)g_records.size() - 1;
}

TimedLaunch::~TimedLaunch() {
  if (index_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (index_ < (int)g_records.size()) hipEventRecord(g_records[index_].stop, stream_);
}

void timing_enable(int on) { g_enabled.store(on ? 1 : 0); }

int timing_count() {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int)g_records.size();
}

int timing_read(int i, const char **name, float *ms) {
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (i < 0 || i >= (int)g_records.size()) return 1;
    *name = g_records[i].name;
    a = g_records[i].start;
    b = g_records[i].stop;
  }
  if (hipEventSynchronize(b) != hipSuccess) return 2;
  return hipEventElapsedTime(ms, a, b) == hipSuccess ? 0 : 2;
}

void timing_reset() {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto &r : g_records) {
    hipEventSynchronize(r.stop);
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
}

}  // namespace kvs
