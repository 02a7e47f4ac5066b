// Attention over the KV cache: the decode kernel (one new query
// per sequence) and the causal prefill kernel (T new queries).
//
// Cache format (FlexGen README, "Extreme Compression": the attention cache is
// stored in 4 bits): per sequence b, head h and position j, head_dim/2 bytes
// of nibble codes and one fp16 {min, scale} pair per 64 channels.  Keys and
// values are reconstructed in registers (fp32 min + code * scale) and never
// written back; the kernel reads 0.5625 bytes per cached element.
//
// Decode, per (b, h) work-group of 256 threads:
//   1. scores: thread t takes positions t, t+256, ...; for each it streams the
//      key's codes (16-byte loads) and computes q . k^ group by group as
//      s_g * (q . c) + min_g * sum(q_g), so the reconstruction costs no extra
//      multiply per element;  scores go to LDS;
//   2. softmax with block max / sum reductions (exp2 of log2(e)-scaled scores);
//   3. values: 16 lanes cover one position's codes (4 bytes = 8 channels per
//      lane), 16 positions are in flight per block; each lane accumulates
//      sum_j (p_j s_jg) c_ji -- two positions at a time, as fp32 dot products
//      of exact fp16 code pairs with the fp16 pair {p_1 s_1, p_2 s_2} -- and
//      sum_j p_j min_jg in fp32, then the 16 partial sums are reduced through
//      LDS.
//
// The fp16 cache (cache compression off, weights possibly still compressed)
// goes through the same kernels instantiated with F16 = true: keys and values
// are read as stored (2 bytes per cached element) instead of reconstructed.
#include <cstdlib>
#include <type_traits>

#include "common.h"

namespace fq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float block_max256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ inline float block_sum256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Codes of 8 consecutive channels (one word) as exact fp16 integers, 4 pairs
// in natural channel order, through the scaled fp8 conversion: the even
// channels' nibbles masked into one byte word, the odd channels' into
// another, two byte permutes pairing them in channel order, and each byte
// read as an OCP e4m3 value (c * 2^-9 for c < 16) scaled by 2^9 -- 9
// instructions per word.
__device__ inline void codes8_cvt(uint32_t w, half2_t out[4]) {
  const uint32_t t = w & 0x0F0F0F0Fu, u = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t p0 = __builtin_amdgcn_perm(u, t, 0x05010400u);  // bytes {c0, c1, c2, c3}
  const uint32_t p1 = __builtin_amdgcn_perm(u, t, 0x07030602u);  // bytes {c4, c5, c6, c7}
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p0, 512.0f, false);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p0, 512.0f, true);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p1, 512.0f, false);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p1, 512.0f, true);
}

// 8 codes (one word) -> the 8 fp16 values fp16(min + c * s), one rounding, as
// 4 packed pairs in channel order: codes8_cvt, then one packed FMA per pair.
__device__ inline void dequant8_cvt(uint32_t w, half2_t mn2, half2_t s2, uint32_t o[4]) {
  half2_t c[4];
  codes8_cvt(w, c);
#pragma unroll
  for (int p = 0; p < 4; ++p) o[p] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c[p], s2, mn2));
}

// Channel k of two positions as an exact fp16 pair {c1_k, c2_k}, for the 8
// channels of code words w1 and w2, through the scaled fp8 conversion: each
// word's even and odd channels' nibbles masked into byte words, one byte
// permute pairing two channels of both positions ({c1_k, c2_k, c1_k', c2_k'}),
// and one conversion per pair -- 18 instructions for 16 codes.
__device__ inline void codes8_pairs(uint32_t w1, uint32_t w2, half2_t out[8]) {
  const uint32_t t1 = w1 & 0x0F0F0F0Fu, u1 = (w1 >> 4) & 0x0F0F0F0Fu;  // channels {0,2,4,6} / {1,3,5,7}
  const uint32_t t2 = w2 & 0x0F0F0F0Fu, u2 = (w2 >> 4) & 0x0F0F0F0Fu;
  const uint32_t e01 = __builtin_amdgcn_perm(t2, t1, 0x05010400u);  // channels 0, 2 of both positions
  const uint32_t e23 = __builtin_amdgcn_perm(t2, t1, 0x07030602u);  // channels 4, 6
  const uint32_t o01 = __builtin_amdgcn_perm(u2, u1, 0x05010400u);  // channels 1, 3
  const uint32_t o23 = __builtin_amdgcn_perm(u2, u1, 0x07030602u);  // channels 5, 7
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e01, 512.0f, false);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e01, 512.0f, true);
  out[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e23, 512.0f, false);
  out[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e23, 512.0f, true);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o01, 512.0f, false);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o01, 512.0f, true);
  out[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o23, 512.0f, false);
  out[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o23, 512.0f, true);
}

// F16 selects the fp16 cache (k16/v16): each position is then covered by D/8
// lanes in both passes, 16 bytes per lane, and the scores are reduced across
// those lanes with xor shuffles.
template <int D, bool F16>
__global__ __launch_bounds__(256) void decode_attention_kernel(const uint16_t* __restrict__ q, int64_t ldq,
                                                               const uint8_t* __restrict__ kc,
                                                               const uint16_t* __restrict__ km,
                                                               const uint8_t* __restrict__ vc,
                                                               const uint16_t* __restrict__ vm, int H, int64_t cap,
                                                               int64_t b0, int len, uint16_t* __restrict__ out,
                                                               int64_t ldo, const uint16_t* __restrict__ k16,
                                                               const uint16_t* __restrict__ v16) {
  constexpr int G = D / 64;       // groups per head
  constexpr int WORDS = D / 8;    // 32-bit code words per position
  constexpr int LPP = WORDS;      // lanes per position in the value pass
  constexpr int SLOTS = 256 / LPP;
  extern __shared__ float smem[];  // [len] probabilities, then [SLOTS][D] partial outputs
  __shared__ float red[4];

  const int b = blockIdx.y, h = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row0 = ((b0 + b) * H + h) * cap;  // first cache row of this (b, h)
  const uint16_t* qp = q + (int64_t)b * ldq + (int64_t)h * D;
  float* p = smem;
  const int slot = tid / LPP, wl = tid % LPP;  // wl: 8-channel chunk of this lane in the per-position passes

  if constexpr (F16) {
    // ---- scores: D/8 lanes per position ----
    const uint4 qr = *reinterpret_cast<const uint4*>(qp + wl * 8);
    const half2_t q2[4] = {__builtin_bit_cast(half2_t, qr.x), __builtin_bit_cast(half2_t, qr.y),
                           __builtin_bit_cast(half2_t, qr.z), __builtin_bit_cast(half2_t, qr.w)};
    float lmax = -INFINITY;
    for (int j = slot; j < len; j += SLOTS) {
      const uint4 kr = *reinterpret_cast<const uint4*>(k16 + (row0 + j) * D + wl * 8);
      float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kr.x), q2[0], 0.f, false);
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kr.y), q2[1], s, false);
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kr.z), q2[2], s, false);
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kr.w), q2[3], s, false);
#pragma unroll
      for (int o = 1; o < LPP; o <<= 1) s += __shfl_xor(s, o);  // the LPP lanes of one position
      s *= kLog2e;
      if (wl == 0) p[j] = s;
      lmax = fmaxf(lmax, s);
    }
    const float mx = block_max256(lmax, red);  // also orders the p[] writes before the reads below
    float lsum = 0.f;
    for (int j = tid; j < len; j += 256) {
      const float e = exp2f(p[j] - mx);
      p[j] = e;
      lsum += e;
    }
    const float inv = 1.0f / block_sum256(lsum, red);
    // ---- values ----
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = slot; j < len; j += SLOTS) {
      const uint4 vr = *reinterpret_cast<const uint4*>(v16 + (row0 + j) * D + wl * 8);
      const uint32_t w[4] = {vr.x, vr.y, vr.z, vr.w};
      const float pj = p[j];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += pj * h2f((uint16_t)(w[k] & 0xFFFF));
        acc[2 * k + 1] += pj * h2f((uint16_t)(w[k] >> 16));
      }
    }
    float* part = smem + ((len + 3) & ~3);
#pragma unroll
    for (int k = 0; k < 8; ++k) part[slot * D + wl * 8 + k] = acc[k];
    __syncthreads();
    if (tid < D) {
      float o = 0.f;
#pragma unroll 4
      for (int s2 = 0; s2 < SLOTS; ++s2) o += part[s2 * D + tid];
      out[(int64_t)b * ldo + (int64_t)h * D + tid] = f2h(o * inv);
    }
    return;
  }

  // ---- query: fp16 pairs in registers, per-group sums of q ----
  half2_t qv[D / 2];
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const uint4 r = *reinterpret_cast<const uint4*>(qp + i * 8);
    qv[4 * i + 0] = __builtin_bit_cast(half2_t, r.x);
    qv[4 * i + 1] = __builtin_bit_cast(half2_t, r.y);
    qv[4 * i + 2] = __builtin_bit_cast(half2_t, r.z);
    qv[4 * i + 3] = __builtin_bit_cast(half2_t, r.w);
  }
  float qsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += (float)qv[g * 32 + i].x + (float)qv[g * 32 + i].y;
    qsum[g] = s;
  }

  // ---- scores: two positions per thread and iteration, both positions'
  // codes requested before either is used (the second clamped to a valid
  // row and discarded when past the end) ----
  float lmax = -INFINITY;
  auto score = [&](const uint4 (&c)[2 * G], const uint32_t (&mb)[G]) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dc = 0.f;
#pragma unroll
      for (int v4 = 0; v4 < 2; ++v4) {
        const uint32_t w[4] = {c[g * 2 + v4].x, c[g * 2 + v4].y, c[g * 2 + v4].z, c[g * 2 + v4].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          half2_t cc[4];
          codes8_cvt(w[k], cc);
          const int base = (g * 64 + v4 * 32 + k * 8) / 2;
#pragma unroll
          for (int u = 0; u < 4; ++u) dc = __builtin_amdgcn_fdot2(cc[u], qv[base + u], dc, false);
        }
      }
      s += h2f((uint16_t)(mb[g] >> 16)) * dc + h2f((uint16_t)(mb[g] & 0xFFFF)) * qsum[g];
    }
    return s * kLog2e;
  };
  for (int j = tid; j < len; j += 512) {
    const int jb = min(j + 256, len - 1);
    const uint4* crow1 = reinterpret_cast<const uint4*>(kc + (row0 + j) * (D / 2));
    const uint4* crow2 = reinterpret_cast<const uint4*>(kc + (row0 + jb) * (D / 2));
    uint4 c1[2 * G], c2[2 * G];
    uint32_t m1[G], m2[G];
#pragma unroll
    for (int i = 0; i < 2 * G; ++i) c1[i] = crow1[i];
#pragma unroll
    for (int i = 0; i < 2 * G; ++i) c2[i] = crow2[i];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m1[g] = reinterpret_cast<const uint32_t*>(km)[(row0 + j) * G + g];
      m2[g] = reinterpret_cast<const uint32_t*>(km)[(row0 + jb) * G + g];
    }
    const float s1 = score(c1, m1);
    p[j] = s1;
    lmax = fmaxf(lmax, s1);
    if (j + 256 < len) {
      const float s2 = score(c2, m2);
      p[j + 256] = s2;
      lmax = fmaxf(lmax, s2);
    }
  }
  // the value pass's first code words are requested before the softmax
  // reductions (they do not depend on the probabilities), and each
  // iteration below requests the next one's before its own arithmetic
  const int g = wl / 8;  // group of this lane's 8 channels
  uint32_t nw1 = 0, nm1 = 0, nw2 = 0, nm2 = 0;
  auto load_v = [&](int j) {
    const int j1 = min(j, len - 1), j2 = min(j + SLOTS, len - 1);  // clamped rows: read, never used
    nw1 = reinterpret_cast<const uint32_t*>(vc + (row0 + j1) * (D / 2))[wl];
    nm1 = reinterpret_cast<const uint32_t*>(vm)[(row0 + j1) * G + g];
    nw2 = reinterpret_cast<const uint32_t*>(vc + (row0 + j2) * (D / 2))[wl];
    nm2 = reinterpret_cast<const uint32_t*>(vm)[(row0 + j2) * G + g];
  };
  load_v(slot);
  const float mx = block_max256(lmax, red);
  float lsum = 0.f;
  for (int j = tid; j < len; j += 256) {
    const float e = exp2f(p[j] - mx);
    p[j] = e;
    lsum += e;
  }
  const float inv = 1.0f / block_sum256(lsum, red);  // also orders the p[] writes before the reads below

  // ---- values ----
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float bsum = 0.f;
  // two positions per iteration: sum_j (p_j s_j) c_jk as fp32 dot products of
  // the fp16 pairs {c_1k, c_2k} and {p_1 s_1, p_2 s_2}
  for (int j = slot; j < len; j += 2 * SLOTS) {
    const int j2 = j + SLOTS;
    const bool two = j2 < len;
    const uint32_t w1 = nw1, mb1 = nm1, w2 = two ? nw2 : 0u, mb2 = two ? nm2 : 0u;
    if (j + 2 * SLOTS < len) load_v(j + 2 * SLOTS);
    const float p1 = p[j], p2 = two ? p[j2] : 0.f;
    bsum += p1 * h2f((uint16_t)(mb1 & 0xFFFF)) + p2 * h2f((uint16_t)(mb2 & 0xFFFF));
    const half2_t a2 = {(half_t)(p1 * h2f((uint16_t)(mb1 >> 16))), (half_t)(p2 * h2f((uint16_t)(mb2 >> 16)))};
    half2_t c[8];
    codes8_pairs(w1, w2, c);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_fdot2(c[k], a2, acc[k], false);
  }
  float* part = smem + ((len + 3) & ~3);
#pragma unroll
  for (int k = 0; k < 8; ++k) part[slot * D + wl * 8 + k] = acc[k] + bsum;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll 4
    for (int s2 = 0; s2 < SLOTS; ++s2) o += part[s2 * D + tid];
    out[(int64_t)b * ldo + (int64_t)h * D + tid] = f2h(o * inv);
  }
}

// ---- causal prefill: flash-style online softmax on the vector units --------
// Block = 64 queries of one (b, h); 4 lanes per query, each owning D/4
// channels.  Keys/values are reconstructed chunk by chunk (64 positions) into
// LDS as fp32 and read back as broadcasts.
template <int D, bool F16>
__global__ __launch_bounds__(256) void prefill_attention_kernel(const uint16_t* __restrict__ q, int64_t ldq,
                                                                const uint8_t* __restrict__ kc,
                                                                const uint16_t* __restrict__ km,
                                                                const uint8_t* __restrict__ vc,
                                                                const uint16_t* __restrict__ vm, int H, int64_t cap,
                                                                int64_t b0, int T, int64_t pos,
                                                                uint16_t* __restrict__ out, int64_t ldo,
                                                                const uint16_t* __restrict__ k16,
                                                                const uint16_t* __restrict__ v16) {
  constexpr int QT = 64, KC = 64, PART = D / 4, G = D / 64;
  __shared__ __attribute__((aligned(16))) float Ks[KC][D + 4];
  __shared__ __attribute__((aligned(16))) float Vs[KC][D + 4];

  const int tid = threadIdx.x;
  const int qi = tid >> 2, part = tid & 3;
  const int b = blockIdx.z, h = blockIdx.y;
  const int t0 = blockIdx.x * QT;
  const int t = t0 + qi;
  const bool qok = t < T;
  const int64_t qpos = pos + t;  // absolute position of this query
  const int64_t row0 = ((b0 + b) * H + h) * cap;

  float qf[PART];
  {
    const uint16_t* qp = q + ((int64_t)b * T + (qok ? t : 0)) * ldq + (int64_t)h * D + part * PART;
#pragma unroll
    for (int i = 0; i < PART; i += 8) {
      const uint4 r = *reinterpret_cast<const uint4*>(qp + i);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qf[i + 2 * k] = h2f((uint16_t)(w[k] & 0xFFFF)) * kLog2e;
        qf[i + 2 * k + 1] = h2f((uint16_t)(w[k] >> 16)) * kLog2e;
      }
    }
  }
  float o[PART];
#pragma unroll
  for (int i = 0; i < PART; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int64_t last_q = pos + min(T, t0 + QT) - 1;  // largest query position in the tile
  const int64_t nkeys = last_q + 1;
  for (int64_t k0 = 0; k0 < nkeys; k0 += KC) {
    __syncthreads();
    // reconstruct KC positions x D channels of K and V: 2*KC*D/8 words over 256 threads
    for (int wi = tid; wi < 2 * KC * (D / 8); wi += 256) {
      const int which = wi / (KC * (D / 8));
      const int r = (wi / (D / 8)) % KC, w8 = wi % (D / 8);
      const int64_t j = k0 + r;
      float* dst = which ? &Vs[r][w8 * 8] : &Ks[r][w8 * 8];
      if constexpr (F16) {
        if (j < nkeys) {
          const uint4 r4 = *reinterpret_cast<const uint4*>((which ? v16 : k16) + (row0 + j) * D + w8 * 8);
          const uint32_t w[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            dst[2 * k] = h2f((uint16_t)(w[k] & 0xFFFF));
            dst[2 * k + 1] = h2f((uint16_t)(w[k] >> 16));
          }
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) dst[k] = 0.f;
        }
      } else if (j < nkeys) {
        const uint8_t* cbase = which ? vc : kc;
        const uint16_t* mbase = which ? vm : km;
        const uint32_t w = reinterpret_cast<const uint32_t*>(cbase + (row0 + j) * (D / 2))[w8];
        const uint32_t mb = reinterpret_cast<const uint32_t*>(mbase)[(row0 + j) * G + w8 / 8];
        const float mn = h2f((uint16_t)(mb & 0xFFFF)), s = h2f((uint16_t)(mb >> 16));
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = mn + (float)((w >> (4 * k)) & 0xF) * s;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = 0.f;
      }
    }
    __syncthreads();
    const int64_t kend = min((int64_t)KC, nkeys - k0);
    for (int r = 0; r < kend; ++r) {
      const int64_t j = k0 + r;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < PART; i += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(&Ks[r][part * PART + i]);
        s += qf[i] * kv.x + qf[i + 1] * kv.y + qf[i + 2] * kv.z + qf[i + 3] * kv.w;
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (!qok || j > qpos) continue;  // causal mask (uniform across the 4 lanes of a query)
      if (s > m) {
        const float c = exp2f(m - s);
        l *= c;
#pragma unroll
        for (int i = 0; i < PART; ++i) o[i] *= c;
        m = s;
      }
      const float pj = exp2f(s - m);
      l += pj;
#pragma unroll
      for (int i = 0; i < PART; i += 4) {
        const float4 vv = *reinterpret_cast<const float4*>(&Vs[r][part * PART + i]);
        o[i] += pj * vv.x;
        o[i + 1] += pj * vv.y;
        o[i + 2] += pj * vv.z;
        o[i + 3] += pj * vv.w;
      }
    }
  }
  if (qok) {
    const float inv = 1.0f / l;
    uint16_t* op = out + ((int64_t)b * T + t) * ldo + (int64_t)h * D + part * PART;
#pragma unroll
    for (int i = 0; i < PART; i += 8) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)f2h(o[i + 2 * k] * inv) | ((uint32_t)f2h(o[i + 2 * k + 1] * inv) << 16);
      *reinterpret_cast<uint4*>(op + i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ---- causal prefill on the matrix cores ------------------------------------
// Work-group = 4 waves x 32 queries of one (b, h); keys in chunks of 64.
// Per chunk the work-group stages K and V of 64 positions in LDS as fp16,
// then each wave computes
//   S^T = K^ Q^T      (v_mfma_f32_16x16x32_f16; lane owns query lane % 16)
//   online softmax    (per query, reduced over the 4 lane groups)
//   O^T += V^T P^T    (P taken straight from the S^T registers)
// With the 4-bit cache each reconstructed key k = min + code * s (exact in
// fp32) is staged as two fp16 arrays, hi = fp16(k) and lo = fp16(k - hi), and
// S^T accumulates the products with both: the scores carry the key to about
// 22 bits instead of fp16's 11 (rounding k itself to fp16 was the largest
// error of the layer at the OPT-175B shape).  V is staged the same way, as
// hi and lo arrays, and O^T accumulates the products with both.
// Transposing both products keeps every per-query value (scores, running
// max/sum, output column) in the lanes of that query, so P never moves.
// V is stored transposed ([d][position]) with the positions of each 32-wide
// slice in the order {0-3, 16-19, 4-7, 20-23, ...}: the order in which a lane
// holds its scores, so the V operand is one 16-byte read per lane.
// LDS rows are 128 bytes with the 16-byte chunk swizzle c ^ (row & 7).
template <int D, bool F16>
__global__ __launch_bounds__(256) void prefill_attention_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ km,
    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vm, int H, int64_t cap, int64_t b0, int T,
    int64_t pos, uint16_t* __restrict__ out, int64_t ldo, const uint16_t* __restrict__ k16,
    const uint16_t* __restrict__ v16) {
  constexpr int KC = 64;           // positions per chunk
  constexpr int NKD = D / 32;      // 32-wide d slices
  constexpr int NDB = D / 16;      // 16-wide d blocks
  constexpr int G = D / 64;        // quantisation groups per position
  constexpr int KHALF = D / 64;    // K stored as D/64 arrays of 64 d (128-byte rows)
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KHALF][KC * 64];
  __shared__ __attribute__((aligned(16))) uint16_t klo_lds[F16 ? 1 : KHALF][F16 ? 8 : KC * 64];  // 4-bit: k - hi
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * KC];
  __shared__ __attribute__((aligned(16))) uint16_t vlo_lds[F16 ? 8 : D * KC];  // 4-bit: v - hi

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int b = blockIdx.z, h = blockIdx.y;
  const int t0 = blockIdx.x * 128 + wave * 32;     // first query of this wave
  const int64_t row0 = ((b0 + b) * H + h) * cap;   // first cache row of this (b, h)
  const int64_t nkeys = pos + min(T, (int)(blockIdx.x * 128 + 128));

  // Q^T operand: lane (query l16 of q-block qb, d slice kd, chunk g4)
  half8_t qf[2][NKD];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = min(t0 + qb * 16 + l16, T - 1);
    const uint16_t* qp = q + ((int64_t)b * T + t) * ldq + (int64_t)h * D;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[qb][kd] = *reinterpret_cast<const half8_t*>(qp + kd * 32 + g4 * 8);
  }
  float4_t oacc[NDB][2];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) oacc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  constexpr float kL2e = 1.4426950408889634f;

  // Staging: every thread stages part of K and part of V of each chunk.
  //   K: key tid / 4, channels (tid % 4) * D/4 .. + D/4 - 1 (D/32 code words);
  //   V: channels 8 * (tid / 16) .. + 7 of the 4 positions of quad tid % 16
  //      (two quads make one 8-position storage chunk in slice order).
  // 4-bit cache: the raw codes and {min, scale} of the next chunk are loaded
  // into registers before the current chunk's products, so their latency
  // hides behind them; they are converted and stored at the next chunk's
  // start.
  constexpr int KW = D / 32;  // K code words (8 channels each) per thread
  const int kkey = tid >> 2, kq = tid & 3;
  const int vdc = tid >> 4, vpq = tid & 15;
  const int vpc = vpq >> 1, vhalf = vpq & 1;  // storage chunk, its first or second 4 positions
  const bool vact = vdc < D / 8;
  auto vkey = [&](int jj) { return (vpc >> 2) * 32 + vhalf * 16 + 4 * (vpc & 3) + jj; };
  uint32_t rk[KW], rkm = 0, rv[4], rvm[4];
  auto load_raw = [&](int64_t k0) {
    if constexpr (!F16) {
      const int64_t j = min(k0 + kkey, nkeys - 1);
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(kc + (row0 + j) * (D / 2)) + kq * KW;
#pragma unroll
      for (int w = 0; w < KW; ++w) rk[w] = cw[w];
      rkm = reinterpret_cast<const uint32_t*>(km)[(row0 + j) * G + (kq * KW * 8) / 64];
      if (vact) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t jv = min(k0 + vkey(jj), nkeys - 1);
          rv[jj] = reinterpret_cast<const uint32_t*>(vc + (row0 + jv) * (D / 2))[vdc];
          rvm[jj] = reinterpret_cast<const uint32_t*>(vm)[(row0 + jv) * G + vdc / 8];
        }
      }
    }
  };
  // 8 codes (one word) with their {min, scale} -> hi = fp16(min + c * s) and
  // lo = fp16((min + c * s) - hi), 4 packed pairs each; min + c * s is exact
  // in fp32 (a 4-bit code times an 11-bit scale), and so is the difference.
  auto hilo8 = [](uint32_t w, uint32_t mb, uint32_t hi[4], uint32_t lo[4]) {
    const float mnf = (float)__builtin_bit_cast(half_t, (uint16_t)(mb & 0xFFFF));
    const float scf = (float)__builtin_bit_cast(half_t, (uint16_t)(mb >> 16));
    half2_t c[4];
    codes8_cvt(w, c);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      half2_t h2, l2;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float v = __builtin_fmaf((float)c[pp][e], scf, mnf);
        h2[e] = (half_t)v;
        l2[e] = (half_t)(v - (float)h2[e]);
      }
      hi[pp] = __builtin_bit_cast(uint32_t, h2);
      lo[pp] = __builtin_bit_cast(uint32_t, l2);
    }
  };
  load_raw(0);
  for (int64_t k0 = 0; k0 < nkeys; k0 += KC) {
    __syncthreads();
    // ---- stage K ----
    {
      const int64_t j = min(k0 + kkey, nkeys - 1);
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        const int d0 = kq * KW * 8 + w * 8;
        const int arr = d0 / 64, chunk = (d0 % 64) / 8;
        const int at = kkey * 64 + ((chunk ^ (kkey & 7)) * 8);
        if constexpr (F16) {
          *reinterpret_cast<uint4*>(&k_lds[arr][at]) = *reinterpret_cast<const uint4*>(k16 + (row0 + j) * D + d0);
        } else {
          uint32_t hi[4], lo[4];
          hilo8(rk[w], rkm, hi, lo);
          *reinterpret_cast<uint4*>(&k_lds[arr][at]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          *reinterpret_cast<uint4*>(&klo_lds[arr][at]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
      }
    }
    // ---- stage V, transposed: [d][positions in slice order] ----
    if (vact) {
      uint32_t hi[4][4], lo[4][4];  // [position][channel pair]
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if constexpr (F16) {
          const int64_t jv = min(k0 + vkey(jj), nkeys - 1);
          const uint4 r4 = *reinterpret_cast<const uint4*>(v16 + (row0 + jv) * D + vdc * 8);
          hi[jj][0] = r4.x, hi[jj][1] = r4.y, hi[jj][2] = r4.z, hi[jj][3] = r4.w;
        } else {
          hilo8(rv[jj], rvm[jj], hi[jj], lo[jj]);
        }
      }
      // channel i: its 4 positions as 8 bytes, the first or second half of a 16-byte chunk
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = vdc * 8 + i;
        const int at = d * KC + ((vpc ^ (d & 7)) * 8) + vhalf * 4;
        auto pick = [&](const uint32_t (*x)[4], int pp) {  // low halves (even channel) or high (odd)
          const uint32_t a = x[2 * pp][i >> 1], c2 = x[2 * pp + 1][i >> 1];
          return (i & 1) ? ((a >> 16) | (c2 & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c2 << 16));
        };
        *reinterpret_cast<uint2*>(&v_lds[at]) = make_uint2(pick(hi, 0), pick(hi, 1));
        if constexpr (!F16) *reinterpret_cast<uint2*>(&vlo_lds[at]) = make_uint2(pick(lo, 0), pick(lo, 1));
      }
    }
    __syncthreads();
    if (k0 + KC < nkeys) load_raw(k0 + KC);
    // skip chunks entirely after this wave's last query (causal)
    if (k0 > pos + t0 + 31) continue;
    // ---- S^T = K^ Q^T : 4 key blocks x 2 query blocks ----
    float4_t sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = (float4_t){0.f, 0.f, 0.f, 0.f};
      const int key = kb * 16 + l16;
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        const int arr = kd / 2, chunk = (kd % 2) * 4 + g4;
        const int at = key * 64 + ((chunk ^ (key & 7)) * 8);
        const half8_t kf = *reinterpret_cast<const half8_t*>(&k_lds[arr][at]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[qb][kd], sacc[kb][qb], 0, 0, 0);
        if constexpr (!F16) {
          const half8_t kl = *reinterpret_cast<const half8_t*>(&klo_lds[arr][at]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qf[qb][kd], sacc[kb][qb], 0, 0, 0);
        }
      }
    }
    // ---- online softmax per query (lane l16 of each query block) ----
    // The exponent base m of a query moves only when its running maximum
    // exceeds m by more than 8 (log2 units): p = 2^(s - m) <= 256 stays well
    // inside fp16, the result is unchanged mathematically (the sum l uses the
    // same base), and the rescale of O is skipped in most chunks (a
    // wave-uniform branch).  Chunks wholly below the wave's first query and
    // inside the keys need no mask.
    const bool unmasked = k0 + KC - 1 <= pos + t0 && k0 + KC <= nkeys;
    half8_t pf[2][2];  // [query block][32-wide key slice], B operand of O^T
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qpos = (int)(pos + t0) + qb * 16 + l16;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = sacc[kb][qb][r] * kL2e;
          if (!unmasked) {
            const int kpos = (int)k0 + kb * 16 + 4 * g4 + r;
            v = (kpos <= qpos && kpos < (int)nkeys) ? v : -INFINITY;
          }
          sacc[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (__any(mx > mrun[qb] + 8.f)) {
        const float mnew = mx > mrun[qb] + 8.f ? mx : mrun[qb];
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun[qb] - mnew);
        lrun[qb] *= alpha;
        mrun[qb] = mnew;
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[i][qb] *= alpha;
      }
      const float mb = mrun[qb] == -INFINITY ? 0.f : mrun[qb];  // a row with no key yet: every p is 0
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(sacc[kb][qb][r] - mb);
          sacc[kb][qb][r] = e;
          sum += e;
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      lrun[qb] += sum;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[qb][sl][r] = (half_t)sacc[2 * sl][qb][r];
          pf[qb][sl][4 + r] = (half_t)sacc[2 * sl + 1][qb][r];
        }
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 16 + l16;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int chunk = sl * 4 + g4;
        const int at = d * KC + ((chunk ^ (d & 7)) * 8);
        const half8_t vf = *reinterpret_cast<const half8_t*>(&v_lds[at]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[qb][sl], oacc[db][qb], 0, 0, 0);
        if constexpr (!F16) {
          const half8_t vl = *reinterpret_cast<const half8_t*>(&vlo_lds[at]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, pf[qb][sl], oacc[db][qb], 0, 0, 0);
        }
      }
    }
  }
  // ---- normalise and store: lane holds channels db*16 + 4*g4 + r of its query ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = t0 + qb * 16 + l16;
    if (t >= T) continue;
    const float inv = 1.0f / lrun[qb];
    uint16_t* op = out + ((int64_t)b * T + t) * ldo + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint32_t w0 = (uint32_t)f2h(oacc[db][qb][0] * inv) | ((uint32_t)f2h(oacc[db][qb][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f2h(oacc[db][qb][2] * inv) | ((uint32_t)f2h(oacc[db][qb][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + db * 16 + 4 * g4) = make_uint2(w0, w1);
    }
  }
}

fq_status check_kv(const fq_kv_layer* kv, const char* who) {
  if (!kv) return fail(FQ_ERR_INVALID, std::string(who) + ": kv is NULL");
  if (kv->group != FQ_GROUP) return fail(FQ_ERR_UNSUPPORTED, std::string(who) + ": only group 64 is implemented");
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(FQ_ERR_UNSUPPORTED, std::string(who) + ": head_dim must be 64 or 128");
  if (!kv_bits_valid(*kv)) return fail(FQ_ERR_INVALID, std::string(who) + ": bits must be 4 or 16");
  if (kv_is_f16(*kv)) {
    if (!kv->k16 || !kv->v16) return fail(FQ_ERR_INVALID, std::string(who) + ": NULL cache buffer");
    if ((uintptr_t)kv->k16 % 16 || (uintptr_t)kv->v16 % 16)
      return fail(FQ_ERR_INVALID, std::string(who) + ": fp16 cache must be 16-byte aligned");
  } else if (!kv->k_codes || !kv->k_meta || !kv->v_codes || !kv->v_meta) {
    return fail(FQ_ERR_INVALID, std::string(who) + ": NULL cache buffer");
  }
  return FQ_OK;
}

// Kernel instantiation for (head_dim, cache format); F(D, F16) launches.
template <typename F>
void by_format(const fq_kv_layer& kv, F&& launch) {
  const bool f16 = kv_is_f16(kv);
  if (kv.head_dim == 128) {
    if (f16) launch(std::integral_constant<int, 128>{}, std::true_type{});
    else launch(std::integral_constant<int, 128>{}, std::false_type{});
  } else {
    if (f16) launch(std::integral_constant<int, 64>{}, std::true_type{});
    else launch(std::integral_constant<int, 64>{}, std::false_type{});
  }
}

}  // namespace
}  // namespace fq

using namespace fq;

// Test hook: FQ_PREFILL_VECTOR=1 in the environment at the time of the call
// selects the vector-unit prefill kernel (fp32 reconstruction) instead of the
// matrix-core one.
static bool prefill_vector_only() {
  const char* e = getenv("FQ_PREFILL_VECTOR");
  return e && e[0] == '1';
}

extern "C" fq_status fq_decode_attention(const uint16_t* q, int64_t ldq, const fq_kv_layer* kv, int64_t b0, int64_t B,
                                         int64_t len, uint16_t* out, int64_t ldo, void* stream) {
  clear_error();
  FQ_TRY(check_kv(kv, "fq_decode_attention"));
  const int64_t hd = (int64_t)kv->heads * kv->head_dim;
  FQ_CHECK_ARG(b0 >= 0 && B >= 0 && b0 + B <= kv->batch, "fq_decode_attention: sequence range exceeds the cache");
  FQ_CHECK_ARG(len >= 1 && len <= kv->capacity, "fq_decode_attention: len must be in [1, capacity]");
  FQ_CHECK_ARG(ldq >= hd && ldo >= hd && ldq % 8 == 0, "fq_decode_attention: bad strides");
  FQ_CHECK_ARG(len <= 30000, "fq_decode_attention: len above 30000 does not fit the LDS score buffer");
  if (B == 0) return FQ_OK;
  FQ_CHECK_ARG(q && out && (uintptr_t)q % 16 == 0, "fq_decode_attention: q/out NULL or q misaligned");
  const int D = kv->head_dim;
  const size_t lds = (size_t)((len + 3) & ~3) * sizeof(float) + (size_t)256 * 8 * sizeof(float);
  const dim3 grid((unsigned)kv->heads, (unsigned)B);
  hipStream_t st = as_stream(stream);
  const int tk = timing_begin(FQ_KC_DECODE_ATTN, st);
  by_format(*kv, [&](auto d, auto f16) {
    decode_attention_kernel<decltype(d)::value, decltype(f16)::value><<<grid, dim3(256), lds, st>>>(
        q, ldq, kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, kv->heads, kv->capacity, b0, (int)len, out, ldo,
        kv->k16, kv->v16);
  });
  FQ_TRY(launch_check("decode_attention_kernel"));
  if (tk >= 0) {
    const double units = (double)B * kv->heads, epb = kv_is_f16(*kv) ? 2.0 : 0.5625;  // cache bytes per element
    timing_end(tk, FQ_KC_DECODE_ATTN, units * 4.0 * len * D, units * (2.0 * len * D * epb + 4.0 * D), st);
  }
  return FQ_OK;
}

extern "C" fq_status fq_prefill_attention(const uint16_t* q, int64_t ldq, const fq_kv_layer* kv, int64_t b0,
                                          int64_t B, int64_t T, int64_t pos, uint16_t* out, int64_t ldo,
                                          void* stream) {
  clear_error();
  FQ_TRY(check_kv(kv, "fq_prefill_attention"));
  const int64_t hd = (int64_t)kv->heads * kv->head_dim;
  FQ_CHECK_ARG(b0 >= 0 && B >= 0 && b0 + B <= kv->batch, "fq_prefill_attention: sequence range exceeds the cache");
  FQ_CHECK_ARG(T >= 0 && pos >= 0 && pos + T <= kv->capacity, "fq_prefill_attention: positions exceed capacity");
  FQ_CHECK_ARG(ldq >= hd && ldo >= hd && ldq % 8 == 0 && ldo % 8 == 0, "fq_prefill_attention: bad strides");
  if (B == 0 || T == 0) return FQ_OK;
  FQ_CHECK_ARG(q && out && (uintptr_t)q % 16 == 0 && (uintptr_t)out % 16 == 0,
               "fq_prefill_attention: q/out NULL or misaligned");
  hipStream_t st = as_stream(stream);
  const int tk = timing_begin(FQ_KC_PREFILL_ATTN, st);
  if (!prefill_vector_only()) {
    const dim3 grid((unsigned)ceil_div(T, 128), (unsigned)kv->heads, (unsigned)B);
    by_format(*kv, [&](auto d, auto f16) {
      prefill_attention_mfma_kernel<decltype(d)::value, decltype(f16)::value><<<grid, dim3(256), 0, st>>>(
          q, ldq, kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, kv->heads, kv->capacity, b0, (int)T, pos, out,
          ldo, kv->k16, kv->v16);
    });
    FQ_TRY(launch_check("prefill_attention_mfma_kernel"));
  } else {
    const dim3 grid((unsigned)ceil_div(T, 64), (unsigned)kv->heads, (unsigned)B);
    by_format(*kv, [&](auto d, auto f16) {
      prefill_attention_kernel<decltype(d)::value, decltype(f16)::value><<<grid, dim3(256), 0, st>>>(
          q, ldq, kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, kv->heads, kv->capacity, b0, (int)T, pos, out,
          ldo, kv->k16, kv->v16);
    });
    FQ_TRY(launch_check("prefill_attention_kernel"));
  }
  if (tk >= 0) {
    const double units = (double)B * kv->heads, d = kv->head_dim, epb = kv_is_f16(*kv) ? 2.0 : 0.5625;
    const double pairs = (double)T * pos + (double)T * (T + 1) / 2.0;  // (query, key) pairs under the causal mask
    timing_end(tk, FQ_KC_PREFILL_ATTN, units * 4.0 * pairs * d, units * (4.0 * T * d + 2.0 * (pos + T) * d * epb),
               st);
  }
  return FQ_OK;
}
