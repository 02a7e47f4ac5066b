// Per-launch HIP-event timing of the library's kernels, grouped by kernel
// class, with the algorithmic work (flops and HBM bytes) of each launch.
// Off by default; when on, every launcher records an event before and after
// its kernel(s) on the caller's stream, so the numbers are device time of
// exactly those launches.
#include <mutex>
#include <vector>

#include "common.h"

namespace fq {
namespace {

struct Record {
  hipEvent_t a, b;
  int cls;
  double flops, bytes;
};

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<Record> recs;    // in use since fq_timing_start
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;  // free event pairs
};

TimingState& state() {
  static TimingState s;
  return s;
}

}  // namespace

int timing_begin(hipStream_t st) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on) return -1;
  Record r{};
  if (!s.pool.empty()) {
    r.a = s.pool.back().first;
    r.b = s.pool.back().second;
    s.pool.pop_back();
  } else if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
    return -1;
  }
  if (hipEventRecord(r.a, st) != hipSuccess) return -1;
  r.cls = -1;
  s.recs.push_back(r);
  return (int)s.recs.size() - 1;
}

void timing_end(int token, int cls, double flops, double bytes, hipStream_t st) {
  if (token < 0) return;
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on || token >= (int)s.recs.size()) return;
  Record& r = s.recs[token];
  r.cls = cls;
  r.flops = flops;
  r.bytes = bytes;
  (void)hipEventRecord(r.b, st);
}

}  // namespace fq

using namespace fq;

extern "C" fq_status fq_timing_start(void) {
  clear_error();
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  for (auto& r : s.recs) s.pool.push_back({r.a, r.b});
  s.recs.clear();
  s.on = true;
  return FQ_OK;
}

extern "C" fq_status fq_timing_stop(fq_kernel_stats* out) {
  clear_error();
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  s.on = false;
  if (out)
    for (int c = 0; c < FQ_KC_COUNT; ++c) out[c] = fq_kernel_stats{0, 0.0, 0.0, 0.0};
  for (auto& r : s.recs) {
    if (r.cls < 0 || r.cls >= FQ_KC_COUNT) continue;
    FQ_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    FQ_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    if (out) {
      out[r.cls].launches += 1;
      out[r.cls].seconds += ms * 1e-3;
      out[r.cls].flops += r.flops;
      out[r.cls].bytes += r.bytes;
    }
  }
  for (auto& r : s.recs) s.pool.push_back({r.a, r.b});
  s.recs.clear();
  return FQ_OK;
}
