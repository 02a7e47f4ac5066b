// Per-launch HIP-event timing of the library's kernels, grouped by kernel
// class, with the algorithmic work (flops and HBM bytes) of each launch.
// Off by default; when on, every launcher of a selected class records an
// event before and after its kernel(s) on the caller's stream, so the numbers
// are device time of exactly those launches.
//
// Events come from a pool that is reused across recording periods and never
// grows past kMaxRecords pairs: launches beyond that are counted as dropped
// and not timed, so a long recording cannot accumulate runtime objects
// without bound.
#include <mutex>
#include <vector>

#include "common.h"

namespace fq {
namespace {

constexpr size_t kMaxRecords = size_t{1} << 16;

struct Record {
  hipEvent_t a, b;
  int cls;
  double flops, bytes;
};

struct TimingState {
  std::mutex mu;
  bool on = false;
  uint32_t mask = 0;
  std::vector<Record> recs;                             // in use since fq_timing_start
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;  // free event pairs
  size_t created = 0;                                   // pairs ever created (<= kMaxRecords)
  int64_t dropped[FQ_KC_COUNT] = {};
};

TimingState& state() {
  static TimingState s;
  return s;
}

}  // namespace

int timing_begin(int cls, hipStream_t st) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on || cls < 0 || cls >= FQ_KC_COUNT || !(s.mask & (1u << cls))) return -1;
  Record r{};
  if (!s.pool.empty()) {
    r.a = s.pool.back().first;
    r.b = s.pool.back().second;
    s.pool.pop_back();
  } else if (s.created < kMaxRecords) {
    if (hipEventCreate(&r.a) != hipSuccess) return -1;
    if (hipEventCreate(&r.b) != hipSuccess) {
      (void)hipEventDestroy(r.a);
      return -1;
    }
    ++s.created;
  } else {
    ++s.dropped[cls];
    return -1;
  }
  if (hipEventRecord(r.a, st) != hipSuccess) {
    s.pool.push_back({r.a, r.b});
    return -1;
  }
  r.cls = -1;  // set when the launch is closed
  s.recs.push_back(r);
  return (int)s.recs.size() - 1;
}

void timing_end(int token, int cls, double flops, double bytes, hipStream_t st) {
  if (token < 0) return;
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on || token >= (int)s.recs.size()) return;
  Record& r = s.recs[token];
  if (hipEventRecord(r.b, st) != hipSuccess) return;
  r.cls = cls;
  r.flops = flops;
  r.bytes = bytes;
}

}  // namespace fq

using namespace fq;

extern "C" fq_status fq_timing_start(uint32_t class_mask) {
  clear_error();
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  for (auto& r : s.recs) s.pool.push_back({r.a, r.b});
  s.recs.clear();
  for (auto& d : s.dropped) d = 0;
  s.mask = class_mask;
  s.on = true;
  return FQ_OK;
}

extern "C" fq_status fq_timing_stop(fq_kernel_stats* out) {
  clear_error();
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  s.on = false;
  if (out)
    for (int c = 0; c < FQ_KC_COUNT; ++c) out[c] = fq_kernel_stats{0, 0.0, 0.0, 0.0, s.dropped[c]};
  fq_status st = FQ_OK;
  for (auto& r : s.recs) {
    if (r.cls < 0 || r.cls >= FQ_KC_COUNT) continue;  // launch failed before its end event
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      st = hip_fail(e, "fq_timing_stop: reading a launch's events");
      break;
    }
    if (out) {
      out[r.cls].launches += 1;
      out[r.cls].seconds += ms * 1e-3;
      out[r.cls].flops += r.flops;
      out[r.cls].bytes += r.bytes;
    }
  }
  for (auto& r : s.recs) s.pool.push_back({r.a, r.b});
  s.recs.clear();
  return st;
}
