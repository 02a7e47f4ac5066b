// Small kernels around the projections: LayerNorm, token + position
// embedding and greedy argmax, the seeded input generator, and the
// library's error state.
#include <cmath>
#include <cstdio>
#include <string>

#include "common.h"

namespace fq {

// ---- error state -------------------------------------------------------------
static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
fq_status fail(fq_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}
fq_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return FQ_ERR_HIP;
}

namespace {

// ---- block reductions (256 threads = 4 waves of 64) ---------------------------
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ---- LayerNorm: one 256-thread block per row, values kept in registers -------
// Each thread owns chunks of 8 consecutive elements (16-byte loads) at stride
// 2048 elements; MAXC chunks cover rows up to 2048*MAXC elements.
template <int MAXC>
__global__ __launch_bounds__(256) void layernorm_kernel(const uint16_t* __restrict__ x, int64_t h, int64_t ldx,
                                                        const uint16_t* __restrict__ gamma,
                                                        const uint16_t* __restrict__ beta, float eps,
                                                        uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  // the row stays in registers as loaded (fp16, converted exactly at each
  // use): half the registers of an fp32 copy, so more rows are in flight per
  // SIMD (the memory stream, not the arithmetic, bounds this kernel)
  uint4 xv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
    if (e < h) {
      xv[c] = *reinterpret_cast<const uint4*>(xr + e);
    }
  }
  auto val = [&](int c, int j) {  // fp16 pair j (elements 2j, 2j+1) of chunk c
    return j < 2 ? (j == 0 ? xv[c].x : xv[c].y) : (j == 2 ? xv[c].z : xv[c].w);
  };
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
    if (e < h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = val(c, j);
        s += h2f((uint16_t)(w & 0xFFFF));
        s += h2f((uint16_t)(w >> 16));
      }
    }
  }
  const float mean = block_sum256(s, red) / (float)h;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
    if (e < h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = val(c, j);
        const float d0 = h2f((uint16_t)(w & 0xFFFF)) - mean, d1 = h2f((uint16_t)(w >> 16)) - mean;
        q += d0 * d0;
        q += d1 * d1;
      }
    }
  }
  const float var = block_sum256(q, red) / (float)h;
  const float rstd = 1.0f / sqrtf(var + eps);
  uint16_t* yr = y + row * ldy;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t e = ((int64_t)c * 256 + threadIdx.x) * 8;
    if (e < h) {
      const uint4 gr = *reinterpret_cast<const uint4*>(gamma + e);
      const uint4 br = *reinterpret_cast<const uint4*>(beta + e);
      const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w};
      const uint32_t bw[4] = {br.x, br.y, br.z, br.w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = val(c, j);
        const float a0 = (h2f((uint16_t)(w & 0xFFFF)) - mean) * rstd * h2f((uint16_t)(gw[j] & 0xFFFF)) +
                         h2f((uint16_t)(bw[j] & 0xFFFF));
        const float a1 = (h2f((uint16_t)(w >> 16)) - mean) * rstd * h2f((uint16_t)(gw[j] >> 16)) +
                         h2f((uint16_t)(bw[j] >> 16));
        o[j] = (uint32_t)f2h(a0) | ((uint32_t)f2h(a1) << 16);
      }
      *reinterpret_cast<uint4*>(yr + e) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// ---- SplitMix64 counter-based generator --------------------------------------
// Steele, Lea, Flood, "Fast Splittable Pseudorandom Number Generators"
// (OOPSLA 2014): output = mix64(state) with state advanced by GAMMA.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void synth_normal_kernel(uint16_t* __restrict__ dst, int64_t n, uint64_t key,
                                                           int64_t first, float scale) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint64_t u = mix64(key + (uint64_t)(first + i + 1) * kGamma);
  const int32_t lane_sum = (int32_t)((u & 0xFFFF) + ((u >> 16) & 0xFFFF) + ((u >> 32) & 0xFFFF) + (u >> 48)) - 131070;
  float prod = (float)lane_sum * scale;
  // The generator is defined as an fp32 product rounded to fp16 (two
  // roundings); keep the compiler from fusing the two into one mixed-
  // precision multiply with a single rounding.
  asm volatile("" : "+v"(prod));
  dst[i] = f2h(prod);
}

__global__ __launch_bounds__(256) void synth_ids_kernel(int32_t* __restrict__ dst, int64_t n, uint64_t key,
                                                        uint32_t vocab) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint64_t u = mix64(key + (uint64_t)(i + 1) * kGamma);
  dst[i] = (int32_t)(((u >> 32) * (uint64_t)vocab) >> 32);
}

__global__ __launch_bounds__(256) void fill_kernel(uint16_t* __restrict__ dst, int64_t n, uint16_t value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = value;
}

// ---- embedding: x[r] = fp16(E[id[r]] + P[pos0 + t + 2]), r = b*T + t ----------
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, int64_t T, int64_t pos0,
                                                    const uint16_t* __restrict__ emb, const uint16_t* __restrict__ pe,
                                                    int64_t h, uint16_t* __restrict__ x) {
  const int64_t r = blockIdx.y;
  const int64_t t = r % T;
  const int64_t id = ids[r];
  const uint16_t* er = emb + id * h;
  const uint16_t* pr = pe + (pos0 + t + 2) * h;
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; e < h; e += (int64_t)gridDim.x * 256 * 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(er + e);
    const uint4 b = *reinterpret_cast<const uint4*>(pr + e);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = h2f((uint16_t)(aw[j] & 0xFFFF)) + h2f((uint16_t)(bw[j] & 0xFFFF));
      const float hi = h2f((uint16_t)(aw[j] >> 16)) + h2f((uint16_t)(bw[j] >> 16));
      o[j] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
    }
    *reinterpret_cast<uint4*>(x + r * h + e) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---- greedy argmax per row, ties to the lowest index -------------------------
__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ logits, int64_t V, int64_t ld,
                                                     int32_t* __restrict__ out) {
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  const float* row = logits + (int64_t)blockIdx.x * ld;
  float best = -INFINITY;
  int32_t bi = 0x7FFFFFFF;
  for (int64_t i = threadIdx.x; i < V; i += 256) {
    const float x = row[i];
    if (x > best) {  // strictly greater: first (lowest) index wins within a thread
      best = x;
      bi = (int32_t)i;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o);
    const int32_t oi = __shfl_xor(bi, o);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = best;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k)
      if (sv[k] > best || (sv[k] == best && si[k] < bi)) {
        best = sv[k];
        bi = si[k];
      }
    out[blockIdx.x] = bi;
  }
}

// y[b] = x[b*T + T-1]: last position of each sequence.
__global__ __launch_bounds__(256) void gather_last_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t h,
                                                          uint16_t* __restrict__ y) {
  const int64_t b = blockIdx.y;
  const uint16_t* src = x + (b * T + T - 1) * h;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < h; e += (int64_t)gridDim.x * 256) y[b * h + e] = src[e];
}

}  // namespace

// ---- launchers ---------------------------------------------------------------
fq_status launch_synth_normal(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream_id, int64_t first,
                              double sigma, hipStream_t st) {
  if (n <= 0) return FQ_OK;
  const uint64_t key = mix64(seed * kGamma + stream_id);
  const double lane_std = std::sqrt((65536.0 * 65536.0 - 1.0) / 3.0);  // std of the 4-lane sum
  const float scale = (float)(sigma / lane_std);
  synth_normal_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st>>>(dst, n, key, first, scale);
  return launch_check("synth_normal_kernel");
}

fq_status launch_fill_f16(uint16_t* dst, int64_t n, uint16_t value, hipStream_t st) {
  if (n <= 0) return FQ_OK;
  fill_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st>>>(dst, n, value);
  return launch_check("fill_kernel");
}

fq_status launch_embed(const int32_t* ids, int64_t rows, int64_t T, int64_t pos0, const uint16_t* emb,
                       const uint16_t* posemb, int64_t h, uint16_t* x, hipStream_t st) {
  if (rows <= 0) return FQ_OK;
  const unsigned gx = (unsigned)ceil_div(h, 2048);
  embed_kernel<<<dim3(gx, (unsigned)rows), dim3(256), 0, st>>>(ids, T, pos0, emb, posemb, h, x);
  return launch_check("embed_kernel");
}

fq_status launch_argmax(const float* logits, int64_t B, int64_t V, int64_t ld, int32_t* out, hipStream_t st) {
  if (B <= 0) return FQ_OK;
  argmax_kernel<<<dim3((unsigned)B), dim3(256), 0, st>>>(logits, V, ld, out);
  return launch_check("argmax_kernel");
}

fq_status launch_gather_rows(const uint16_t* x, int64_t B, int64_t T, int64_t h, uint16_t* y, hipStream_t st) {
  if (B <= 0) return FQ_OK;
  gather_last_kernel<<<dim3((unsigned)ceil_div(h, 256 * 8), (unsigned)B), dim3(256), 0, st>>>(x, T, h, y);
  return launch_check("gather_last_kernel");
}

}  // namespace fq

using namespace fq;

extern "C" const char* fq_last_error(void) { return g_last_error.c_str(); }
extern "C" const char* fq_version(void) { return "libfq 0.1 (gfx950)"; }

extern "C" fq_status fq_layernorm(const uint16_t* x, int64_t M, int64_t h, int64_t ldx, const uint16_t* gamma,
                                  const uint16_t* beta, float eps, uint16_t* y, int64_t ldy, void* stream) {
  clear_error();
  FQ_CHECK_ARG(M >= 0 && h > 0, "fq_layernorm: bad shape");
  FQ_CHECK_ARG(h % 8 == 0 && ldx % 8 == 0 && ldy % 8 == 0, "fq_layernorm: h and strides must be multiples of 8");
  FQ_CHECK_ARG(ldx >= h && ldy >= h, "fq_layernorm: stride < h");
  FQ_CHECK_ARG(h <= 2048 * 8, "fq_layernorm: h above 16384 is not supported");
  if (M == 0) return FQ_OK;
  FQ_CHECK_ARG(x && gamma && beta && y, "fq_layernorm: NULL buffer");
  FQ_CHECK_ARG(((uintptr_t)x | (uintptr_t)y | (uintptr_t)gamma | (uintptr_t)beta) % 16 == 0,
               "fq_layernorm: buffers must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  const dim3 grid((unsigned)M);
  const int tk = timing_begin(FQ_KC_LAYERNORM, st);
  if (h <= 2048)
    layernorm_kernel<1><<<grid, dim3(256), 0, st>>>(x, h, ldx, gamma, beta, eps, y, ldy);
  else if (h <= 4096)
    layernorm_kernel<2><<<grid, dim3(256), 0, st>>>(x, h, ldx, gamma, beta, eps, y, ldy);
  else if (h <= 8192)
    layernorm_kernel<4><<<grid, dim3(256), 0, st>>>(x, h, ldx, gamma, beta, eps, y, ldy);
  else
    layernorm_kernel<8><<<grid, dim3(256), 0, st>>>(x, h, ldx, gamma, beta, eps, y, ldy);
  FQ_TRY(launch_check("layernorm_kernel"));
  timing_end(tk, FQ_KC_LAYERNORM, 0.0, (double)M * h * 4.0 + 4.0 * h, st);
  return FQ_OK;
}

extern "C" fq_status fq_synth_normal_f16(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream_id, int64_t first,
                                         double sigma, void* stream) {
  clear_error();
  FQ_CHECK_ARG(n >= 0 && first >= 0, "fq_synth_normal_f16: negative size");
  if (n == 0) return FQ_OK;
  FQ_CHECK_ARG(dst != nullptr, "fq_synth_normal_f16: dst is NULL");
  return launch_synth_normal(dst, n, seed, stream_id, first, sigma, as_stream(stream));
}

extern "C" fq_status fq_synth_token_ids(int32_t* dst, int64_t n, uint64_t seed, uint64_t stream_id, int32_t vocab,
                                        void* stream) {
  clear_error();
  FQ_CHECK_ARG(n >= 0 && vocab > 0, "fq_synth_token_ids: bad size");
  if (n == 0) return FQ_OK;
  FQ_CHECK_ARG(dst != nullptr, "fq_synth_token_ids: dst is NULL");
  const uint64_t key = mix64(seed * kGamma + stream_id);
  synth_ids_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, as_stream(stream)>>>(dst, n, key,
                                                                                          (uint32_t)vocab);
  return launch_check("synth_ids_kernel");
}
