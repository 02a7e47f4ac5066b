// Runtime of libfq: model and KV-cache handles, the decoder-layer step, the
// greedy generation loop, and layer-by-layer weight streaming from pinned
// host memory.
//
// Pages: FlexGen README (giters.com mirror) -- "Extreme Compression" (4-bit
// weights and cache), "Benchmark Results" (prompt 512, output 32; throughput
// = generated tokens / (prompt time + generation time)), the block schedule
// that reuses each loaded weight across the whole batch and overlaps I/O with
// compute, "Get Started" (--percent placement of weights), "Handle Out-of-
// memory" (--compress-weight, --pin-weight); awesome-repositories feature
// list, "Asynchronous Tensor Loading" (weights copied from host memory while
// the current layer computes).
//
// Schedule.  Prefill is layer-major: each layer is applied to every chunk of
// sequences before the next layer starts, so a streamed layer is copied once
// per pass and serves the whole batch (the block schedule).  Streamed layers
// (fp16, or packed 4-bit codes + {min, scale} when weights are compressed:
// 3.56x fewer bytes over the host link) use two device staging buffers: a
// copy stream fills buffer (l+1)%2 while the compute stream runs layer l from
// buffer l%2; events copied[s] and consumed[s] order the two streams (no
// host waits).
#include <algorithm>
#include <chrono>
#include <cmath>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "common.h"

// Streams of the seeded generator (one per tensor): per-layer tensor t of
// layer l uses stream l*64 + t; model-level tensors use 2^20 + k.
namespace {
enum { T_WQKV = 0, T_WOUT, T_WFC1, T_WFC2, T_BQKV, T_BOUT, T_BFC1, T_BFC2, T_LN1G, T_LN1B, T_LN2G, T_LN2B };
constexpr uint64_t S_EMBED = (1u << 20) + 2, S_POS = (1u << 20) + 3, S_LNFG = (1u << 20) + 4,
                   S_LNFB = (1u << 20) + 5;
constexpr uint16_t kOneF16 = 0x3C00;
}  // namespace

struct LayerStore {
  fq_packed w[4] = {};           // packed weights (compress_weight)
  uint16_t* w16[4] = {};         // resident fp16 weights
  uint16_t* small = nullptr;     // device: b_qkv | b_out | b_fc1 | b_fc2 | ln1_g | ln1_b | ln2_g | ln2_b
  int host_blob = -1;            // streamed: index of the host blob holding this layer
};

struct fq_model {
  fq_model_config cfg{};
  fq_policy pol{};
  int device = 0;
  std::vector<LayerStore> layers;
  // model-level parameters
  uint16_t* embed = nullptr;
  uint16_t* pos = nullptr;
  uint16_t* lnf = nullptr;  // gamma | beta
  // activation workspace (max_tokens rows)
  int64_t max_tokens = 0;
  uint16_t *h1 = nullptr, *qkv = nullptr, *att = nullptr, *x1 = nullptr, *f = nullptr;
  // streaming
  std::vector<uint8_t*> host_blobs;  // pinned host, one layer each (fp16 or packed)
  uint8_t* stage[2] = {nullptr, nullptr};
  hipStream_t copy_stream = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr};
  hipEvent_t consumed[2] = {nullptr, nullptr};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> copy_ev;  // per-copy timing events
  size_t n_copies = 0;
  int staged[2] = {-1, -1};
  double h2d_bytes = 0, h2d_s = 0;
  // generation buffers (grown on demand)
  uint16_t* gen_x = nullptr;
  size_t gen_x_bytes = 0;
  float* logits = nullptr;
  size_t logits_bytes = 0;
  int32_t* ids = nullptr;
  size_t ids_bytes = 0;
  std::vector<void*> allocs;
  std::vector<fq_capture> captures;  // parity-test hook (fq_model_set_capture)

  int64_t h() const { return cfg.hidden; }
  int64_t F() const { return cfg.ffn; }
  int64_t d() const { return cfg.hidden / cfg.heads; }
  int64_t layer_elems() const { return 4 * h() * h() + 2 * h() * F(); }
  int64_t small_elems() const { return 3 * h() + h() + F() + h() + 4 * h(); }
  // bytes of one layer's weights as stored in a host blob / staging buffer:
  // fp16, or packed codes + {min, scale} (0.5625 byte per weight)
  size_t blob_bytes() const {
    return pol.compress_weight ? (size_t)layer_elems() / 2 + (size_t)layer_elems() / 64 * 4
                               : (size_t)layer_elems() * 2;
  }
  bool streamed(int l) const { return layers[l].host_blob >= 0; }
};

// One buffer per layer, laid out [k codes | v codes | k meta | v meta] (4-bit)
// or [k | v] (fp16), each tensor [batch, heads, capacity, per-position bytes].
struct fq_kv {
  int layers = 0;
  std::vector<fq_kv_layer> views;  // device views; host views for offloaded layers
  std::vector<void*> allocs;
  int device = 0;
  // offloaded layers (pinned host memory, staged through two device buffers)
  std::vector<uint8_t*> host;  // per layer: host buffer or nullptr (resident)
  uint8_t* stage[2] = {nullptr, nullptr};
  fq_kv_layer stage_view[2] = {};
  int staged[2] = {-1, -1};
  size_t layer_bytes = 0;
  hipStream_t copy_stream = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr}, consumed[2] = {nullptr, nullptr};
  double h2d_bytes = 0, d2h_bytes = 0;
  bool offloaded(int l) const { return host[l] != nullptr; }
};

using namespace fq;

namespace {

fq_status dmalloc(fq_model* m, void** p, size_t bytes, const char* what) {
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(FQ_ERR_OOM, std::string("device allocation failed: ") + what + " (" + std::to_string(bytes) + " bytes)");
  }
  m->allocs.push_back(*p);
  return FQ_OK;
}

// Weight slices of one layer inside an fp16 blob [qkv | out | fc1 | fc2].
void blob_slices(const fq_model* m, uint16_t* base, uint16_t* w[4]) {
  const int64_t h = m->h(), F = m->F();
  w[0] = base;
  w[1] = w[0] + 3 * h * h;
  w[2] = w[1] + h * h;
  w[3] = w[2] + F * h;
}

void weight_shape(const fq_model* m, int which, int64_t* n, int64_t* k);

// Packed weights of one layer inside a blob [codes qkv | meta qkv | codes out
// | meta out | codes fc1 | meta fc1 | codes fc2 | meta fc2] (every part a
// multiple of 256 bytes, so each keeps the GEMM's 16-byte alignment).
void packed_slices(const fq_model* m, uint8_t* base, fq_packed w[4]) {
  uint8_t* cur = base;
  for (int k = 0; k < 4; ++k) {
    int64_t n, kk;
    weight_shape(m, k, &n, &kk);
    w[k].rows = n;
    w[k].cols = kk;
    w[k].group = FQ_GROUP;
    w[k].codes = cur;
    cur += (size_t)n * kk / 2;
    w[k].meta = reinterpret_cast<uint16_t*>(cur);
    cur += (size_t)n * (kk / 64) * 4;
  }
}

void weight_shape(const fq_model* m, int which, int64_t* n, int64_t* k) {
  const int64_t h = m->h(), F = m->F();
  const int64_t N[4] = {3 * h, h, F, h}, K[4] = {h, h, h, F};
  *n = N[which];
  *k = K[which];
}

// Device weight operand of layer l: its resident copy, or the slice of the
// staging buffer its host blob was copied into.
fq_weight layer_weight(const fq_model* m, int l, int which, uint8_t* staged) {
  fq_weight w{};
  weight_shape(m, which, &w.n, &w.k);
  if (m->pol.compress_weight) {
    w.kind = FQ_WEIGHT_PACKED4;
    if (staged) {
      fq_packed p[4];
      packed_slices(m, staged, p);
      w.packed = p[which];
    } else {
      w.packed = m->layers[l].w[which];
    }
  } else {
    w.kind = FQ_WEIGHT_F16;
    if (staged) {
      uint16_t* p[4];
      blob_slices(m, reinterpret_cast<uint16_t*>(staged), p);
      w.w16 = p[which];
    } else {
      w.w16 = m->layers[l].w16[which];
    }
  }
  return w;
}

// Rows of sequences [b0, b0+B) x T tokens (row = b*T + t, stride `ld`
// elements) copied to a capture buffer [nb, capacity, h] at positions
// pos..pos+T-1, for the sequences the capture holds.
fq_status capture_rows(const fq_capture& c, uint16_t* dst, const uint16_t* src, int64_t ld, int64_t h, int64_t b0,
                       int64_t B, int64_t T, int64_t pos, hipStream_t st) {
  if (!dst) return FQ_OK;
  const int64_t s0 = std::max(b0, c.b0), s1 = std::min(b0 + B, c.b0 + c.nb);
  if (s0 >= s1) return FQ_OK;
  if (pos + T > c.capacity) return fail(FQ_ERR_INVALID, "capture: positions beyond the capture's capacity");
  for (int64_t s = s0; s < s1; ++s)
    FQ_HIP(hipMemcpy2DAsync(dst + ((s - c.b0) * c.capacity + pos) * h, (size_t)h * 2, src + (s - b0) * T * ld,
                            (size_t)ld * 2, (size_t)h * 2, (size_t)T, hipMemcpyDeviceToDevice, st));
  return FQ_OK;
}

const fq_capture* find_capture(const fq_model* m, int l) {
  for (const fq_capture& c : m->captures)
    if (c.layer == l) return &c;
  return nullptr;
}

// The core of one decoder layer over M = B*T rows (see fq_layer_step).
fq_status layer_compute(fq_model* m, int l, const fq_kv_layer& kv, int64_t b0, int64_t B, int64_t T, int64_t pos,
                        const uint16_t* x, uint16_t* y, uint8_t* staged, hipStream_t st) {
  const int64_t h = m->h(), F = m->F(), M = B * T;
  const uint16_t* sp = m->layers[l].small;
  const uint16_t *b_qkv = sp, *b_out = sp + 3 * h, *b_fc1 = b_out + h, *b_fc2 = b_fc1 + F;
  const uint16_t *ln1g = b_fc2 + h, *ln1b = ln1g + h, *ln2g = ln1b + h, *ln2b = ln2g + h;
  const fq_weight wq = layer_weight(m, l, 0, staged), wo = layer_weight(m, l, 1, staged),
                  w1 = layer_weight(m, l, 2, staged), w2 = layer_weight(m, l, 3, staged);
  void* s = (void*)st;
  const fq_capture* cap = find_capture(m, l);
  if (cap) FQ_TRY(capture_rows(*cap, cap->x_in, x, h, h, b0, B, T, pos, st));
  FQ_TRY(fq_layernorm(x, M, h, h, ln1g, ln1b, 1e-5f, m->h1, h, s));
  const float qscale = 1.0f / std::sqrt((float)m->d());
  if (!cap) {
    // QKV projection; K/V go to the cache (quantised in the GEMM epilogue at prefill sizes)
    FQ_TRY(fq_qkv_gemm_append(m->h1, M, h, &wq, b_qkv, qscale, &kv, b0, B, T, pos, m->qkv, 3 * h, s));
  } else {
    // the same results in two calls (the fused call is defined as equal to
    // them bit for bit), so that K and V exist in fp16 and can be recorded
    FQ_TRY(fq_dequant_gemm(m->h1, M, h, &wq, b_qkv, nullptr, 0, FQ_EPI_BIAS | FQ_EPI_QSCALE, qscale, h, m->qkv,
                           3 * h, s));
    FQ_TRY(fq_kv_append(&kv, m->qkv + h, m->qkv + 2 * h, 3 * h, b0, B, T, pos, s));
    FQ_TRY(capture_rows(*cap, cap->k16, m->qkv + h, 3 * h, h, b0, B, T, pos, st));
    FQ_TRY(capture_rows(*cap, cap->v16, m->qkv + 2 * h, 3 * h, h, b0, B, T, pos, st));
  }
  if (T == 1)
    FQ_TRY(fq_decode_attention(m->qkv, 3 * h, &kv, b0, B, pos + 1, m->att, h, s));
  else
    FQ_TRY(fq_prefill_attention(m->qkv, 3 * h, &kv, b0, B, T, pos, m->att, h, s));
  FQ_TRY(fq_dequant_gemm(m->att, M, h, &wo, b_out, x, h, FQ_EPI_BIAS | FQ_EPI_RESIDUAL, 1.f, 0, m->x1, h, s));
  if (cap) FQ_TRY(capture_rows(*cap, cap->x1, m->x1, h, h, b0, B, T, pos, st));
  FQ_TRY(fq_layernorm(m->x1, M, h, h, ln2g, ln2b, 1e-5f, m->h1, h, s));
  FQ_TRY(fq_dequant_gemm(m->h1, M, h, &w1, b_fc1, nullptr, 0, FQ_EPI_BIAS | FQ_EPI_RELU, 1.f, 0, m->f, F, s));
  FQ_TRY(fq_dequant_gemm(m->f, M, F, &w2, b_fc2, m->x1, h, FQ_EPI_BIAS | FQ_EPI_RESIDUAL, 1.f, 0, y, h, s));
  if (cap) FQ_TRY(capture_rows(*cap, cap->y_out, y, h, h, b0, B, T, pos, st));
  return FQ_OK;
}

// ---- streaming -------------------------------------------------------------
// Issue the copy of layer l's host blob into staging slot l%2 on the copy
// stream, after the compute stream has released that slot (event consumed).
// Each copy records its own pair of timing events, read after the pass.
fq_status stream_issue(fq_model* m, int l) {
  const int slot = l & 1;
  if (m->staged[slot] == l) return FQ_OK;
  const size_t bytes = m->blob_bytes();
  if (m->n_copies == m->copy_ev.size()) {
    hipEvent_t a, b;
    FQ_HIP(hipEventCreate(&a));
    FQ_HIP(hipEventCreate(&b));
    m->copy_ev.push_back({a, b});
  }
  const auto& ev = m->copy_ev[m->n_copies++];
  FQ_HIP(hipStreamWaitEvent(m->copy_stream, m->consumed[slot], 0));
  FQ_HIP(hipEventRecord(ev.first, m->copy_stream));
  FQ_HIP(hipMemcpyAsync(m->stage[slot], m->host_blobs[m->layers[l].host_blob], bytes, hipMemcpyHostToDevice,
                        m->copy_stream));
  FQ_HIP(hipEventRecord(ev.second, m->copy_stream));
  FQ_HIP(hipEventRecord(m->copied[slot], m->copy_stream));
  m->staged[slot] = l;
  m->h2d_bytes += (double)bytes;
  return FQ_OK;
}

// Sum the copy intervals recorded since the last call (host waits for them).
fq_status stream_collect(fq_model* m) {
  for (size_t i = 0; i < m->n_copies; ++i) {
    float ms = 0.f;
    FQ_HIP(hipEventSynchronize(m->copy_ev[i].second));
    FQ_HIP(hipEventElapsedTime(&ms, m->copy_ev[i].first, m->copy_ev[i].second));
    m->h2d_s += ms * 1e-3;
  }
  m->n_copies = 0;
  return FQ_OK;
}

// ---- cache offload ----------------------------------------------------------
// Copy positions [p0, p1) of sequences [b0, b1) (every head, K and V, codes
// and meta) between two buffers of one layer's cache layout: one strided copy
// per tensor (rows = (sequence, head) pairs, pitch = capacity positions).
// `dst` and `src` are views of the same shape and format.
fq_status kv_copy_positions(const fq_kv_layer& dst, const fq_kv_layer& src, int64_t b0, int64_t b1, int64_t p0,
                            int64_t p1, hipMemcpyKind kind, hipStream_t st, double* bytes) {
  if (p1 <= p0 || b1 <= b0) return FQ_OK;
  const int64_t H = dst.heads, cap = dst.capacity, d = dst.head_dim;
  struct T {
    const void* src;
    void* dst;
    size_t e;  // bytes per (sequence, head, position)
  };
  std::vector<T> ts;
  if (kv_is_f16(dst)) {
    ts = {{src.k16, dst.k16, (size_t)d * 2}, {src.v16, dst.v16, (size_t)d * 2}};
  } else {
    ts = {{src.k_codes, dst.k_codes, (size_t)d / 2}, {src.v_codes, dst.v_codes, (size_t)d / 2},
          {src.k_meta, dst.k_meta, (size_t)(d / 64) * 4}, {src.v_meta, dst.v_meta, (size_t)(d / 64) * 4}};
  }
  for (const T& t : ts) {
    const size_t pitch = (size_t)cap * t.e, off = (size_t)b0 * H * pitch + (size_t)p0 * t.e;
    const size_t width = (size_t)(p1 - p0) * t.e, height = (size_t)(b1 - b0) * H;
    FQ_HIP(hipMemcpy2DAsync((uint8_t*)t.dst + off, pitch, (const uint8_t*)t.src + off, pitch, width, height, kind,
                            st));
    *bytes += (double)width * height;
  }
  return FQ_OK;
}

// Stage offloaded layer l into slot l%2 on the cache copy stream: positions
// [0, pos) of sequences [0, B) (the prefix the pass reads; the new positions
// are written by the layer itself), after the slot's previous layer has been
// written back (event consumed).
fq_status kv_issue(fq_kv* kv, int l, int64_t B, int64_t pos) {
  const int slot = l & 1;
  if (kv->staged[slot] == l) return FQ_OK;
  FQ_HIP(hipStreamWaitEvent(kv->copy_stream, kv->consumed[slot], 0));
  FQ_TRY(kv_copy_positions(kv->stage_view[slot], kv->views[l], 0, B, 0, pos, hipMemcpyHostToDevice,
                           kv->copy_stream, &kv->h2d_bytes));
  FQ_HIP(hipEventRecord(kv->copied[slot], kv->copy_stream));
  kv->staged[slot] = l;
  return FQ_OK;
}

// After layer l computed on `st`: write positions [pos, pos+T) back to host
// memory on the copy stream and release the slot.
fq_status kv_writeback(fq_kv* kv, int l, int64_t B, int64_t T, int64_t pos, hipStream_t st) {
  const int slot = l & 1;
  FQ_HIP(hipEventRecord(kv->done[slot], st));
  FQ_HIP(hipStreamWaitEvent(kv->copy_stream, kv->done[slot], 0));
  FQ_TRY(kv_copy_positions(kv->views[l], kv->stage_view[slot], 0, B, pos, pos + T, hipMemcpyDeviceToHost,
                           kv->copy_stream, &kv->d2h_bytes));
  FQ_HIP(hipEventRecord(kv->consumed[slot], kv->copy_stream));
  return FQ_OK;
}

// Run layers 0..L-1 over groups of at most cs sequences (layer-major, so a
// streamed layer is copied once per pass and reused by every group).  x holds
// B*T rows and is updated in place.
fq_status run_layers(fq_model* m, fq_kv* kv, int64_t B, int64_t T, int64_t pos, uint16_t* x, int64_t cs,
                     hipStream_t st) {
  const int L = m->cfg.layers;
  const int64_t h = m->h();
  kv->staged[0] = kv->staged[1] = -1;  // staged caches are valid within one pass only
  for (int l = 0; l < L; ++l) {
    uint8_t* sp = nullptr;
    if (m->streamed(l)) {
      const int slot = l & 1;
      FQ_TRY(stream_issue(m, l));  // no-op when prefetched during layer l-1
      FQ_HIP(hipStreamWaitEvent(st, m->copied[slot], 0));
      sp = m->stage[slot];
    }
    const fq_kv_layer* view = &kv->views[l];
    if (kv->offloaded(l)) {
      FQ_TRY(kv_issue(kv, l, B, pos));
      FQ_HIP(hipStreamWaitEvent(st, kv->copied[l & 1], 0));
      view = &kv->stage_view[l & 1];
    }
    // prefetch layer l+1 (weights, cache) into the other slots while layer l computes
    if (m->pol.overlap && l + 1 < L && m->streamed(l + 1)) FQ_TRY(stream_issue(m, l + 1));
    if (m->pol.overlap && l + 1 < L && kv->offloaded(l + 1)) FQ_TRY(kv_issue(kv, l + 1, B, pos));
    for (int64_t b0 = 0; b0 < B; b0 += cs) {
      const int64_t nb = std::min(cs, B - b0);
      uint16_t* xc = x + b0 * T * h;
      FQ_TRY(layer_compute(m, l, *view, b0, nb, T, pos, xc, xc, sp, st));
    }
    if (m->streamed(l)) FQ_HIP(hipEventRecord(m->consumed[l & 1], st));
    if (kv->offloaded(l)) FQ_TRY(kv_writeback(kv, l, B, T, pos, st));
  }
  return FQ_OK;
}

fq_status grow(fq_model* m, void** p, size_t* have, size_t need, const char* what) {
  if (*have >= need) return FQ_OK;
  if (*p) {
    FQ_HIP(hipDeviceSynchronize());
    auto it = std::find(m->allocs.begin(), m->allocs.end(), *p);
    if (it != m->allocs.end()) m->allocs.erase(it);
    (void)hipFree(*p);
    *p = nullptr;
    *have = 0;
  }
  FQ_TRY(dmalloc(m, p, need, what));
  *have = need;
  return FQ_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
extern "C" fq_status fq_model_create(const fq_model_config* cfg, const fq_policy* policy, fq_model** out) {
  clear_error();
  FQ_CHECK_ARG(cfg && policy && out, "fq_model_create: NULL argument");
  *out = nullptr;
  FQ_CHECK_ARG(cfg->hidden > 0 && cfg->heads > 0 && cfg->ffn > 0 && cfg->layers > 0, "fq_model_create: bad sizes");
  FQ_CHECK_ARG(cfg->hidden % cfg->heads == 0, "fq_model_create: hidden must be a multiple of heads");
  const int d = cfg->hidden / cfg->heads;
  if (d != 64 && d != 128) return fail(FQ_ERR_UNSUPPORTED, "fq_model_create: head_dim must be 64 or 128");
  FQ_CHECK_ARG(cfg->hidden % 64 == 0 && cfg->ffn % 64 == 0, "fq_model_create: hidden and ffn must be multiples of 64");
  FQ_CHECK_ARG(cfg->vocab >= 0 && (cfg->vocab == 0 || cfg->max_pos > 2), "fq_model_create: bad vocab/max_pos");
  FQ_CHECK_ARG(policy->resident_layers >= -1, "fq_model_create: bad resident_layers");
  FQ_CHECK_ARG(policy->host_layers >= 0, "fq_model_create: bad host_layers");

  fq_model* m = new (std::nothrow) fq_model();
  if (!m) return fail(FQ_ERR_OOM, "fq_model_create: host allocation failed");
  m->cfg = *cfg;
  m->pol = *policy;
  m->max_tokens = policy->max_tokens > 0 ? policy->max_tokens : 16384;
  hipError_t ge = hipGetDevice(&m->device);
  if (ge != hipSuccess) {
    delete m;
    return hip_fail(ge, "hipGetDevice");
  }
  auto bail = [&](fq_status s) {
    std::string msg = fq_last_error();
    fq_model_destroy(m);
    return fail(s, msg);
  };
  const int L = cfg->layers;
  const int64_t h = m->h(), F = m->F();
  m->layers.resize(L);
  const int resident = policy->resident_layers < 0 ? L : std::min(L, policy->resident_layers);
  const int streamed = L - resident;
  const int nblobs = streamed == 0 ? 0 : (policy->host_layers > 0 ? std::min(streamed, policy->host_layers) : streamed);
  for (int l = 0; l < L; ++l) {
    LayerStore& ls = m->layers[l];
    fq_status s;
    if (l >= resident) {
      ls.host_blob = (l - resident) % nblobs;
    } else if (policy->compress_weight) {
      uint8_t* blob = nullptr;
      if ((s = dmalloc(m, (void**)&blob, m->blob_bytes(), "packed layer")) != FQ_OK) return bail(s);
      packed_slices(m, blob, ls.w);
    } else {
      uint16_t* blob = nullptr;
      if ((s = dmalloc(m, (void**)&blob, m->blob_bytes(), "fp16 layer")) != FQ_OK) return bail(s);
      blob_slices(m, blob, ls.w16);
    }
    if ((s = dmalloc(m, (void**)&ls.small, (size_t)m->small_elems() * 2, "layer vectors")) != FQ_OK) return bail(s);
  }
  fq_status s;
  if (cfg->vocab > 0) {
    if ((s = dmalloc(m, (void**)&m->embed, (size_t)cfg->vocab * h * 2, "embedding")) != FQ_OK) return bail(s);
    if ((s = dmalloc(m, (void**)&m->pos, (size_t)cfg->max_pos * h * 2, "positions")) != FQ_OK) return bail(s);
    if ((s = dmalloc(m, (void**)&m->lnf, (size_t)2 * h * 2, "final LN")) != FQ_OK) return bail(s);
  }
  const int64_t mt = m->max_tokens;
  if ((s = dmalloc(m, (void**)&m->h1, (size_t)mt * h * 2, "workspace")) != FQ_OK) return bail(s);
  if ((s = dmalloc(m, (void**)&m->qkv, (size_t)mt * 3 * h * 2, "workspace")) != FQ_OK) return bail(s);
  if ((s = dmalloc(m, (void**)&m->att, (size_t)mt * h * 2, "workspace")) != FQ_OK) return bail(s);
  if ((s = dmalloc(m, (void**)&m->x1, (size_t)mt * h * 2, "workspace")) != FQ_OK) return bail(s);
  if ((s = dmalloc(m, (void**)&m->f, (size_t)mt * F * 2, "workspace")) != FQ_OK) return bail(s);
  if (nblobs > 0) {
    m->host_blobs.assign(nblobs, nullptr);
    for (int i = 0; i < nblobs; ++i) {
      hipError_t e = hipHostMalloc((void**)&m->host_blobs[i], m->blob_bytes(), hipHostMallocDefault);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        m->host_blobs[i] = nullptr;
        return bail(fail(FQ_ERR_OOM, "fq_model_create: pinned host allocation failed"));
      }
    }
    for (int k = 0; k < 2; ++k) {
      if ((s = dmalloc(m, (void**)&m->stage[k], m->blob_bytes(), "staging")) != FQ_OK) return bail(s);
      if (hipEventCreateWithFlags(&m->copied[k], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&m->consumed[k], hipEventDisableTiming) != hipSuccess)
        return bail(fail(FQ_ERR_HIP, "fq_model_create: event creation failed"));
    }
    if (hipStreamCreateWithFlags(&m->copy_stream, hipStreamNonBlocking) != hipSuccess)
      return bail(fail(FQ_ERR_HIP, "fq_model_create: copy stream creation failed"));
  }
  *out = m;
  return FQ_OK;
}

extern "C" fq_status fq_model_destroy(fq_model* m) {
  if (!m) return FQ_OK;
  (void)hipDeviceSynchronize();
  for (void* p : m->allocs) (void)hipFree(p);
  for (uint8_t* p : m->host_blobs)
    if (p) (void)hipHostFree(p);
  for (int k = 0; k < 2; ++k) {
    if (m->copied[k]) (void)hipEventDestroy(m->copied[k]);
    if (m->consumed[k]) (void)hipEventDestroy(m->consumed[k]);
  }
  for (auto& e : m->copy_ev) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  if (m->copy_stream) (void)hipStreamDestroy(m->copy_stream);
  delete m;
  return FQ_OK;
}

namespace {

// Store one layer's fp16 parameters (device pointers) into the model.
fq_status set_layer(fq_model* m, int l, const fq_layer_weights* w, hipStream_t st) {
  const int64_t h = m->h(), F = m->F();
  LayerStore& ls = m->layers[l];
  const uint16_t* src[4] = {w->w_qkv, w->w_out, w->w_fc1, w->w_fc2};
  fq_packed staged[4];
  // The staging slots may hold a copy of this layer (or of another layer that
  // shares its host blob): forget both, so that the next pass copies the new
  // weights in.
  m->staged[0] = m->staged[1] = -1;
  if (m->pol.compress_weight && ls.host_blob >= 0) {
    // quantise into staging slot 0 (no generation is running), then copy the
    // packed layer to its host blob
    FQ_HIP(hipDeviceSynchronize());
    packed_slices(m, m->stage[0], staged);
  }
  for (int k = 0; k < 4; ++k) {
    int64_t n, kk;
    weight_shape(m, k, &n, &kk);
    if (m->pol.compress_weight) {
      FQ_TRY(fq_quantize(src[k], n, kk, kk, ls.host_blob >= 0 ? &staged[k] : &ls.w[k], (void*)st));
    } else if (ls.host_blob < 0) {
      FQ_HIP(hipMemcpyAsync(ls.w16[k], src[k], (size_t)n * kk * 2, hipMemcpyDeviceToDevice, st));
    } else {
      uint16_t* hw[4];
      blob_slices(m, reinterpret_cast<uint16_t*>(m->host_blobs[ls.host_blob]), hw);
      FQ_HIP(hipMemcpyAsync(hw[k], src[k], (size_t)n * kk * 2, hipMemcpyDeviceToHost, st));
    }
  }
  if (m->pol.compress_weight && ls.host_blob >= 0)
    FQ_HIP(hipMemcpyAsync(m->host_blobs[ls.host_blob], m->stage[0], m->blob_bytes(), hipMemcpyDeviceToHost, st));
  const uint16_t* vec[8] = {w->b_qkv, w->b_out, w->b_fc1, w->b_fc2, w->ln1_g, w->ln1_b, w->ln2_g, w->ln2_b};
  const int64_t len[8] = {3 * h, h, F, h, h, h, h, h};
  uint16_t* dst = ls.small;
  for (int k = 0; k < 8; ++k) {
    FQ_HIP(hipMemcpyAsync(dst, vec[k], (size_t)len[k] * 2, hipMemcpyDeviceToDevice, st));
    dst += len[k];
  }
  return FQ_OK;
}

}  // namespace

extern "C" fq_status fq_model_set_layer(fq_model* m, int32_t layer, const fq_layer_weights* w, void* stream) {
  clear_error();
  FQ_CHECK_ARG(m && w, "fq_model_set_layer: NULL argument");
  FQ_CHECK_ARG(layer >= 0 && layer < m->cfg.layers, "fq_model_set_layer: layer out of range");
  FQ_CHECK_ARG(w->w_qkv && w->w_out && w->w_fc1 && w->w_fc2 && w->b_qkv && w->b_out && w->b_fc1 && w->b_fc2 &&
                   w->ln1_g && w->ln1_b && w->ln2_g && w->ln2_b,
               "fq_model_set_layer: NULL parameter");
  hipStream_t st = as_stream(stream);
  FQ_TRY(set_layer(m, layer, w, st));
  if (m->layers[layer].host_blob >= 0) FQ_HIP(hipStreamSynchronize(st));
  return FQ_OK;
}

extern "C" fq_status fq_model_set_embeddings(fq_model* m, const uint16_t* embed, const uint16_t* pos,
                                             const uint16_t* lnf_g, const uint16_t* lnf_b, void* stream) {
  clear_error();
  FQ_CHECK_ARG(m && embed && pos && lnf_g && lnf_b, "fq_model_set_embeddings: NULL argument");
  FQ_CHECK_ARG(m->cfg.vocab > 0, "fq_model_set_embeddings: model has no vocabulary");
  const int64_t h = m->h();
  hipStream_t st = as_stream(stream);
  FQ_HIP(hipMemcpyAsync(m->embed, embed, (size_t)m->cfg.vocab * h * 2, hipMemcpyDeviceToDevice, st));
  FQ_HIP(hipMemcpyAsync(m->pos, pos, (size_t)m->cfg.max_pos * h * 2, hipMemcpyDeviceToDevice, st));
  FQ_HIP(hipMemcpyAsync(m->lnf, lnf_g, (size_t)h * 2, hipMemcpyDeviceToDevice, st));
  FQ_HIP(hipMemcpyAsync(m->lnf + h, lnf_b, (size_t)h * 2, hipMemcpyDeviceToDevice, st));
  return FQ_OK;
}

extern "C" fq_status fq_model_init_random(fq_model* m, uint64_t seed, double bias_sigma, void* stream) {
  clear_error();
  FQ_CHECK_ARG(m != nullptr, "fq_model_init_random: NULL model");
  hipStream_t st = as_stream(stream);
  const int64_t h = m->h(), F = m->F();
  // one fp16 layer of scratch for the generated weights
  uint16_t* scratch = nullptr;
  hipError_t e = hipMalloc(&scratch, (size_t)(m->layer_elems() + m->small_elems()) * 2);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FQ_ERR_OOM, "fq_model_init_random: scratch allocation failed");
  }
  fq_status rs = FQ_OK;
  auto run = [&]() -> fq_status {
    std::vector<int> done_blob(m->host_blobs.size(), 0);
    for (int l = 0; l < m->cfg.layers; ++l) {
      const int blob = m->layers[l].host_blob;
      if (blob >= 0 && done_blob[blob]) continue;  // shared host blob already filled
      uint16_t* w[4];
      blob_slices(m, scratch, w);
      const uint64_t base = (uint64_t)l * 64;
      for (int k = 0; k < 4; ++k) {
        int64_t n, kk;
        weight_shape(m, k, &n, &kk);
        FQ_TRY(launch_synth_normal(w[k], n * kk, seed, base + T_WQKV + k, 0, 0.02, st));
      }
      uint16_t* v = scratch + m->layer_elems();
      const int64_t len[8] = {3 * h, h, F, h, h, h, h, h};
      const int tid[8] = {T_BQKV, T_BOUT, T_BFC1, T_BFC2, T_LN1G, T_LN1B, T_LN2G, T_LN2B};
      uint16_t* vp[8];
      uint16_t* cur = v;
      for (int k = 0; k < 8; ++k) {
        vp[k] = cur;
        const bool gamma = (tid[k] == T_LN1G || tid[k] == T_LN2G);
        if (bias_sigma > 0)
          FQ_TRY(launch_synth_normal(cur, len[k], seed, base + tid[k], 0, gamma ? 1.0 : bias_sigma, st));
        else
          FQ_TRY(launch_fill_f16(cur, len[k], gamma ? kOneF16 : 0, st));
        cur += len[k];
      }
      fq_layer_weights lw{w[0], w[1], w[2], w[3], vp[0], vp[1], vp[2], vp[3], vp[4], vp[5], vp[6], vp[7]};
      FQ_TRY(set_layer(m, l, &lw, st));
      if (blob >= 0) done_blob[blob] = 1;
      FQ_HIP(hipStreamSynchronize(st));  // scratch is reused by the next layer
    }
    // layers sharing a host blob take the vectors of the layer that filled it
    for (int l = 0; l < m->cfg.layers; ++l) {
      const int blob = m->layers[l].host_blob;
      if (blob < 0) continue;
      for (int l2 = 0; l2 < l; ++l2)
        if (m->layers[l2].host_blob == blob) {
          FQ_HIP(hipMemcpyAsync(m->layers[l].small, m->layers[l2].small, (size_t)m->small_elems() * 2,
                                hipMemcpyDeviceToDevice, st));
          break;
        }
    }
    if (m->cfg.vocab > 0) {
      FQ_TRY(launch_synth_normal(m->embed, (int64_t)m->cfg.vocab * h, seed, S_EMBED, 0, 0.02, st));
      FQ_TRY(launch_synth_normal(m->pos, (int64_t)m->cfg.max_pos * h, seed, S_POS, 0, 0.02, st));
      if (bias_sigma > 0) {
        FQ_TRY(launch_synth_normal(m->lnf, h, seed, S_LNFG, 0, 1.0, st));
        FQ_TRY(launch_synth_normal(m->lnf + h, h, seed, S_LNFB, 0, bias_sigma, st));
      } else {
        FQ_TRY(launch_fill_f16(m->lnf, h, kOneF16, st));
        FQ_TRY(launch_fill_f16(m->lnf + h, h, 0, st));
      }
    }
    FQ_HIP(hipStreamSynchronize(st));
    return FQ_OK;
  };
  rs = run();
  (void)hipStreamSynchronize(st);
  (void)hipFree(scratch);
  return rs;
}

extern "C" fq_status fq_model_packed_weight(const fq_model* m, int32_t layer, int32_t which, fq_packed* out) {
  clear_error();
  FQ_CHECK_ARG(m && out, "fq_model_packed_weight: NULL argument");
  FQ_CHECK_ARG(layer >= 0 && layer < m->cfg.layers && which >= 0 && which < 4, "fq_model_packed_weight: bad index");
  if (!m->pol.compress_weight) return fail(FQ_ERR_INVALID, "fq_model_packed_weight: weights are not compressed");
  if (m->layers[layer].host_blob >= 0)
    return fail(FQ_ERR_INVALID, "fq_model_packed_weight: layer is streamed from host memory");
  *out = m->layers[layer].w[which];
  return FQ_OK;
}

extern "C" fq_status fq_model_set_capture(fq_model* m, const fq_capture* caps, int32_t n) {
  clear_error();
  FQ_CHECK_ARG(m != nullptr, "fq_model_set_capture: NULL model");
  FQ_CHECK_ARG(n >= 0 && n <= 8 && (n == 0 || caps), "fq_model_set_capture: between 0 and 8 captures");
  for (int32_t i = 0; i < n; ++i) {
    const fq_capture& c = caps[i];
    FQ_CHECK_ARG(c.layer >= 0 && c.layer < m->cfg.layers, "fq_model_set_capture: layer out of range");
    FQ_CHECK_ARG(c.b0 >= 0 && c.nb > 0 && c.capacity > 0, "fq_model_set_capture: bad sequence range or capacity");
    for (int32_t j = 0; j < i; ++j)
      FQ_CHECK_ARG(caps[j].layer != c.layer, "fq_model_set_capture: one capture per layer");
  }
  m->captures.assign(caps, caps + n);
  return FQ_OK;
}

namespace {
// View of one layer's cache inside a buffer of the layout described at fq_kv.
fq_kv_layer kv_view_at(uint8_t* base, bool f16, int64_t batch, int H, int64_t d, int64_t capacity) {
  const size_t codes = (size_t)batch * H * capacity * d / 2;
  const size_t meta = (size_t)batch * H * capacity * (d / 64) * 4;
  const size_t elems = (size_t)batch * H * capacity * d;
  fq_kv_layer v{};
  if (f16) {
    v.bits = 16;
    v.k16 = reinterpret_cast<uint16_t*>(base);
    v.v16 = reinterpret_cast<uint16_t*>(base) + elems;
  } else {
    v.bits = 4;
    v.k_codes = base;
    v.v_codes = base + codes;
    v.k_meta = reinterpret_cast<uint16_t*>(base + 2 * codes);
    v.v_meta = reinterpret_cast<uint16_t*>(base + 2 * codes + meta);
  }
  v.batch = batch;
  v.heads = H;
  v.head_dim = (int32_t)d;
  v.capacity = capacity;
  v.group = FQ_GROUP;
  return v;
}
}  // namespace

extern "C" fq_status fq_kv_create(const fq_model* m, int64_t batch, int64_t capacity, fq_kv** out) {
  clear_error();
  FQ_CHECK_ARG(m && out, "fq_kv_create: NULL argument");
  FQ_CHECK_ARG(batch > 0 && capacity > 0, "fq_kv_create: bad size");
  FQ_CHECK_ARG(m->pol.cache_resident_layers >= -1, "fq_kv_create: bad cache_resident_layers");
  *out = nullptr;
  fq_kv* kv = new (std::nothrow) fq_kv();
  if (!kv) return fail(FQ_ERR_OOM, "fq_kv_create: host allocation failed");
  kv->layers = m->cfg.layers;
  kv->device = m->device;
  const int H = m->cfg.heads;
  const int64_t d = m->d();
  const bool f16 = !m->pol.compress_cache;
  const size_t elems = (size_t)batch * H * capacity * d;
  kv->layer_bytes = f16 ? 2 * elems * 2 : 2 * (elems / 2 + elems / 64 * 4);
  const int L = kv->layers;
  const int resident = m->pol.cache_resident_layers < 0 ? L : std::min(L, m->pol.cache_resident_layers);
  auto bail = [&](fq_status s, const char* msg) {
    fq_kv_destroy(kv);
    return fail(s, msg);
  };
  kv->host.assign(L, nullptr);
  for (int l = 0; l < L; ++l) {
    uint8_t* base = nullptr;
    if (l < resident) {
      if (hipMalloc(&base, kv->layer_bytes) != hipSuccess) {
        (void)hipGetLastError();
        return bail(FQ_ERR_OOM, "fq_kv_create: device allocation failed");
      }
      kv->allocs.push_back(base);
    } else {
      if (hipHostMalloc((void**)&base, kv->layer_bytes, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        return bail(FQ_ERR_OOM, "fq_kv_create: pinned host allocation failed");
      }
      kv->host[l] = base;
    }
    kv->views.push_back(kv_view_at(base, f16, batch, H, d, capacity));
  }
  if (resident < L) {
    for (int k = 0; k < 2; ++k) {
      if (hipMalloc(&kv->stage[k], kv->layer_bytes) != hipSuccess) {
        (void)hipGetLastError();
        kv->stage[k] = nullptr;
        return bail(FQ_ERR_OOM, "fq_kv_create: staging allocation failed");
      }
      kv->stage_view[k] = kv_view_at(kv->stage[k], f16, batch, H, d, capacity);
      if (hipEventCreateWithFlags(&kv->copied[k], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&kv->done[k], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&kv->consumed[k], hipEventDisableTiming) != hipSuccess)
        return bail(FQ_ERR_HIP, "fq_kv_create: event creation failed");
    }
    if (hipStreamCreateWithFlags(&kv->copy_stream, hipStreamNonBlocking) != hipSuccess)
      return bail(FQ_ERR_HIP, "fq_kv_create: copy stream creation failed");
  }
  *out = kv;
  return FQ_OK;
}

extern "C" fq_status fq_kv_destroy(fq_kv* kv) {
  if (!kv) return FQ_OK;
  (void)hipDeviceSynchronize();
  for (void* p : kv->allocs) (void)hipFree(p);
  for (uint8_t* p : kv->host)
    if (p) (void)hipHostFree(p);
  for (int k = 0; k < 2; ++k) {
    if (kv->stage[k]) (void)hipFree(kv->stage[k]);
    for (hipEvent_t e : {kv->copied[k], kv->done[k], kv->consumed[k]})
      if (e) (void)hipEventDestroy(e);
  }
  if (kv->copy_stream) (void)hipStreamDestroy(kv->copy_stream);
  delete kv;
  return FQ_OK;
}

extern "C" fq_status fq_kv_layer_view(const fq_kv* kv, int32_t layer, fq_kv_layer* out) {
  clear_error();
  FQ_CHECK_ARG(kv && out, "fq_kv_layer_view: NULL argument");
  FQ_CHECK_ARG(layer >= 0 && layer < kv->layers, "fq_kv_layer_view: layer out of range");
  *out = kv->views[layer];
  return FQ_OK;
}

extern "C" fq_status fq_layer_step(fq_model* m, int32_t layer, fq_kv* kv, int64_t b0, int64_t B, int64_t T,
                                   int64_t pos, const uint16_t* x, uint16_t* y, void* stream) {
  clear_error();
  FQ_CHECK_ARG(m && kv, "fq_layer_step: NULL handle");
  FQ_CHECK_ARG(layer >= 0 && layer < m->cfg.layers && layer < kv->layers, "fq_layer_step: layer out of range");
  FQ_CHECK_ARG(b0 >= 0 && B >= 0 && T >= 0 && pos >= 0, "fq_layer_step: negative index");
  FQ_CHECK_ARG(B * T <= m->max_tokens, "fq_layer_step: B*T exceeds the policy's max_tokens");
  const fq_kv_layer& v = kv->views[layer];
  FQ_CHECK_ARG(v.heads == m->cfg.heads && v.head_dim == m->d(), "fq_layer_step: cache does not match the model");
  FQ_CHECK_ARG(b0 + B <= v.batch && pos + T <= v.capacity, "fq_layer_step: cache too small");
  if (B == 0 || T == 0) return FQ_OK;
  FQ_CHECK_ARG(x && y && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0, "fq_layer_step: x/y NULL or misaligned");
  hipStream_t st = as_stream(stream);
  uint8_t* sp = nullptr;
  if (m->streamed(layer)) {
    // synchronous staging of a host-resident layer into slot 0
    FQ_HIP(hipMemcpyAsync(m->stage[0], m->host_blobs[m->layers[layer].host_blob], m->blob_bytes(),
                          hipMemcpyHostToDevice, st));
    m->staged[0] = -1;
    sp = m->stage[0];
  }
  if (!kv->offloaded(layer)) return layer_compute(m, layer, v, b0, B, T, pos, x, y, sp, st);
  // offloaded cache: stage the prefix of these sequences into slot 0, run the
  // layer, write the new positions back, all on `stream`, then wait
  FQ_HIP(hipStreamSynchronize(kv->copy_stream));
  double bytes = 0;
  FQ_TRY(kv_copy_positions(kv->stage_view[0], v, b0, b0 + B, 0, pos, hipMemcpyHostToDevice, st, &bytes));
  kv->staged[0] = -1;
  FQ_TRY(layer_compute(m, layer, kv->stage_view[0], b0, B, T, pos, x, y, sp, st));
  FQ_TRY(kv_copy_positions(v, kv->stage_view[0], b0, b0 + B, pos, pos + T, hipMemcpyDeviceToHost, st, &bytes));
  FQ_HIP(hipStreamSynchronize(st));
  return FQ_OK;
}

namespace {
fq_progress_fn g_progress = nullptr;
void* g_progress_user = nullptr;
}  // namespace

extern "C" void fq_set_progress(fq_progress_fn fn, void* user) {
  g_progress = fn;
  g_progress_user = user;
}

extern "C" fq_status fq_generate(fq_model* m, fq_kv* kv, const int32_t* prompt_ids, int64_t B, int64_t P,
                                 int64_t gen_len, int32_t* out_ids, float* logits, fq_gen_stats* stats, void* stream) {
  clear_error();
  FQ_CHECK_ARG(m && kv && prompt_ids && out_ids, "fq_generate: NULL argument");
  FQ_CHECK_ARG(m->cfg.vocab > 0, "fq_generate: model has no vocabulary");
  FQ_CHECK_ARG(B > 0 && P > 0 && gen_len > 0, "fq_generate: bad sizes");
  FQ_CHECK_ARG(kv->layers == m->cfg.layers, "fq_generate: cache layer count differs");
  FQ_CHECK_ARG(B <= kv->views[0].batch, "fq_generate: batch exceeds the cache");
  FQ_CHECK_ARG(P + gen_len - 1 <= kv->views[0].capacity, "fq_generate: prompt + generation exceeds cache capacity");
  FQ_CHECK_ARG(P + gen_len + 1 <= m->cfg.max_pos, "fq_generate: position table too short");
  FQ_CHECK_ARG(B <= m->max_tokens && P <= m->max_tokens, "fq_generate: batch or prompt exceeds max_tokens");
  for (int64_t i = 0; i < B * P; ++i)
    FQ_CHECK_ARG(prompt_ids[i] >= 0 && prompt_ids[i] < m->cfg.vocab, "fq_generate: prompt id out of range");
  hipStream_t st = as_stream(stream);
  const int64_t h = m->h(), V = m->cfg.vocab;
  const int64_t cs = std::max<int64_t>(1, std::min<int64_t>(B, m->max_tokens / P));  // sequences per prefill chunk
  FQ_TRY(grow(m, (void**)&m->gen_x, &m->gen_x_bytes, (size_t)B * P * h * 2, "activations"));
  FQ_TRY(grow(m, (void**)&m->logits, &m->logits_bytes, (size_t)B * V * 4, "logits"));
  FQ_TRY(grow(m, (void**)&m->ids, &m->ids_bytes, (size_t)(B * P + B * gen_len) * 4, "token ids"));
  int32_t* d_prompt = m->ids;
  int32_t* d_out = m->ids + B * P;
  m->h2d_bytes = 0;
  m->h2d_s = 0;
  m->n_copies = 0;
  // staged copies are trusted within one generation only (the caller may
  // replace layers between calls)
  m->staged[0] = m->staged[1] = -1;
  kv->h2d_bytes = kv->d2h_bytes = 0;

  hipEvent_t ev[3];
  for (int i = 0; i < 3; ++i) FQ_HIP(hipEventCreate(&ev[i]));
  const fq_progress_fn progress = g_progress;
  void* const progress_user = g_progress_user;
  std::vector<hipEvent_t> step_ev;
  int64_t reported = 0;  // steps reported to `progress`
  if (progress) {
    step_ev.resize(gen_len);
    for (auto& e : step_ev) FQ_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  auto run = [&]() -> fq_status {
    FQ_HIP(hipEventRecord(ev[0], st));
    FQ_HIP(hipMemcpyAsync(d_prompt, prompt_ids, (size_t)B * P * 4, hipMemcpyHostToDevice, st));
    uint16_t* x = m->gen_x;
    FQ_TRY(launch_embed(d_prompt, B * P, P, 0, m->embed, m->pos, h, x, st));
    FQ_TRY(run_layers(m, kv, B, P, 0, x, cs, st));
    fq_weight head{};
    head.kind = FQ_WEIGHT_F16;
    head.w16 = m->embed;
    head.n = V;
    head.k = h;
    for (int64_t step = 0; step < gen_len; ++step) {
      // last position of each sequence -> final LN -> logits -> argmax
      const int64_t T = step == 0 ? P : 1;
      uint16_t* xl = x;
      if (T > 1) {
        FQ_TRY(launch_gather_rows(x, B, T, h, m->att, st));
        xl = m->att;
      }
      FQ_TRY(fq_layernorm(xl, B, h, h, m->lnf, m->lnf + h, 1e-5f, m->h1, h, (void*)st));
      float* lg = logits ? logits + step * B * V : m->logits;
      FQ_TRY(fq_dequant_gemm(m->h1, B, h, &head, nullptr, nullptr, 0, FQ_EPI_F32OUT, 1.f, 0, lg, V, (void*)st));
      FQ_TRY(launch_argmax(lg, B, V, V, d_out + step * B, st));
      if (step == 0) FQ_HIP(hipEventRecord(ev[1], st));
      if (progress) {
        FQ_HIP(hipEventRecord(step_ev[step], st));
        // queueing is paced by the device once its queue is full: report the
        // steps already finished (non-blocking query, in order)
        while (reported < step && hipEventQuery(step_ev[reported]) == hipSuccess) {
          ++reported;
          progress(reported, gen_len, progress_user);
        }
      }
      if (step + 1 == gen_len) break;
      const int64_t pos = P + step;  // position of the token just generated
      FQ_TRY(launch_embed(d_out + step * B, B, 1, pos, m->embed, m->pos, h, x, st));
      FQ_TRY(run_layers(m, kv, B, 1, pos, x, B, st));
    }
    FQ_HIP(hipEventRecord(ev[2], st));
    for (; progress && reported < gen_len; ++reported) {
      FQ_HIP(hipEventSynchronize(step_ev[reported]));
      progress(reported + 1, gen_len, progress_user);
    }
    FQ_HIP(hipEventSynchronize(ev[2]));
    if (kv->copy_stream) FQ_HIP(hipStreamSynchronize(kv->copy_stream));  // last write-backs
    FQ_TRY(stream_collect(m));
    // d_out is [gen_len, B]; out_ids is [B, gen_len]
    std::vector<int32_t> tmp((size_t)gen_len * B);
    FQ_HIP(hipMemcpy(tmp.data(), d_out, tmp.size() * 4, hipMemcpyDeviceToHost));
    for (int64_t s = 0; s < gen_len; ++s)
      for (int64_t b = 0; b < B; ++b) out_ids[b * gen_len + s] = tmp[s * B + b];
    if (stats) {
      float t01 = 0.f, t12 = 0.f;
      FQ_HIP(hipEventElapsedTime(&t01, ev[0], ev[1]));
      FQ_HIP(hipEventElapsedTime(&t12, ev[1], ev[2]));
      stats->prefill_s = t01 * 1e-3;
      stats->decode_s = t12 * 1e-3;
      stats->tokens_per_s = (double)B * gen_len / (stats->prefill_s + stats->decode_s);
      stats->h2d_bytes = m->h2d_bytes;
      stats->h2d_s = m->h2d_s;
      stats->kv_h2d_bytes = kv->h2d_bytes;
      stats->kv_d2h_bytes = kv->d2h_bytes;
    }
    return FQ_OK;
  };
  fq_status s = run();
  for (int i = 0; i < 3; ++i) (void)hipEventDestroy(ev[i]);
  for (auto& e : step_ev) (void)hipEventDestroy(e);
  return s;
}
