// Host-side memory and undefined-behaviour check of the generation path.
//
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// of every library source (the device code is built normally; see build.sh)
// and run on a GPU: small greedy generations (FlexGen README, "Benchmark
// Results": prompt in, generated tokens out) through each host path of
// fq_generate -- weights resident, 4-bit layers streamed from pinned host
// memory with and without copy overlap, fp16 layers streamed, the KV cache
// of some layers offloaded -- each inside a per-launch timing window, then
// one timing window driven past the event pool's cap.  Any sanitizer report
// ends the run with a nonzero status; otherwise it prints one line per case
// and "host sanitizer driver: ok".
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fq.h"

namespace {

bool ok(fq_status s, const char* what) {
  if (s == FQ_OK) return true;
  std::fprintf(stderr, "%s failed: status %d: %s\n", what, (int)s, fq_last_error());
  return false;
}

struct Case {
  const char* name;
  int compress_weight, compress_cache, resident_layers, host_layers, overlap, cache_resident_layers;
};

// One model: create, initialise, generate with every kernel class timed, destroy.
bool run_case(const Case& c, int reps, bool expect_drop) {
  const fq_model_config cfg = {256, 4, 1024, 4, 512, 128};
  fq_policy pol = {};
  pol.compress_weight = c.compress_weight;
  pol.compress_cache = c.compress_cache;
  pol.resident_layers = c.resident_layers;
  pol.host_layers = c.host_layers;
  pol.overlap = c.overlap;
  pol.max_tokens = 256;  // 8 x 64 prompt rows: two prefill chunks
  pol.cache_resident_layers = c.cache_resident_layers;
  const int64_t B = 8, P = 64, G = 8;
  fq_model* m = nullptr;
  fq_kv* kv = nullptr;
  if (!ok(fq_model_create(&cfg, &pol, &m), "fq_model_create")) return false;
  bool good = ok(fq_model_init_random(m, 7, 0.02, nullptr), "fq_model_init_random") &&
              ok(fq_kv_create(m, B, P + G - 1, &kv), "fq_kv_create");
  std::vector<int32_t> ids(B * P), out(B * G), first(B * G);
  uint32_t s = 12345;
  for (auto& v : ids) v = (int32_t)((s = s * 1664525u + 1013904223u) >> 23);  // < 512
  fq_kernel_stats st[FQ_KC_COUNT];
  if (good) good = ok(fq_timing_start(FQ_KC_ALL), "fq_timing_start");
  fq_gen_stats gs = {};
  for (int r = 0; good && r < reps; ++r) {
    good = ok(fq_generate(m, kv, ids.data(), B, P, G, out.data(), nullptr, &gs, nullptr), "fq_generate");
    if (good && r == 0) first = out;
    if (good && out != first) {
      std::fprintf(stderr, "%s: generation %d differs from the first\n", c.name, r);
      good = false;
    }
  }
  if (good) good = ok(fq_timing_stop(st), "fq_timing_stop");
  if (good) {
    int64_t launches = 0, dropped = 0;
    for (int k = 0; k < FQ_KC_COUNT; ++k) launches += st[k].launches, dropped += st[k].dropped;
    std::printf("%-28s reps %3d  tokens/s %9.1f  timed launches %6lld  dropped %6lld  h2d %.3g B  kv h2d %.3g B\n",
                c.name, reps, gs.tokens_per_s, (long long)launches, (long long)dropped, gs.h2d_bytes,
                gs.kv_h2d_bytes);
    if (expect_drop && dropped == 0) {
      std::fprintf(stderr, "%s: expected launches beyond the timing pool\n", c.name);
      good = false;
    }
  }
  if (kv) good = ok(fq_kv_destroy(kv), "fq_kv_destroy") && good;
  good = ok(fq_model_destroy(m), "fq_model_destroy") && good;
  return good;
}

}  // namespace

int main() {
  std::setvbuf(stdout, nullptr, _IONBF, 0);
  const Case cases[] = {
      {"resident 4-bit", 1, 1, -1, 0, 1, -1},
      {"streamed 4-bit, overlap", 1, 1, 1, 0, 1, -1},
      {"streamed 4-bit, no overlap", 1, 1, 2, 0, 0, -1},
      {"streamed fp16, shared blobs", 0, 1, 1, 2, 1, -1},
      {"cache offloaded", 1, 1, -1, 0, 1, 2},
      {"fp16 cache, fp16 weights", 0, 0, -1, 0, 1, -1},
  };
  for (const Case& c : cases)
    if (!run_case(c, 2, false)) return 1;
  // one timing window past the 65536-launch pool (about 250 launches per generation)
  if (!run_case(cases[0], 300, true)) return 1;
  std::printf("host sanitizer driver: ok\n");
  // End here, before the static destructors: the HIP runtime's own exit-time
  // teardown frees memory after the sanitizer's device-allocator hooks have
  // been unloaded, which trips an internal sanitizer CHECK (runtime code, not
  // this library's).
  std::_Exit(0);
}
