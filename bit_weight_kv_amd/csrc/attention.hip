// Attention over the KV cache: the decode kernel (one new query
// per sequence) and the causal prefill kernel (T new queries).
//
// Cache format (FlexGen README, "Extreme Compression": the attention cache is
// stored in 4 bits): per sequence b, head h and position j, head_dim/2 bytes
// of nibble codes and one fp16 {min, scale} pair per 64 channels.  Keys and
// values are reconstructed in registers (fp32 min + code * scale) and never
// written back; the kernel reads 0.5625 bytes per cached element.
//
// Decode, per (b, h) work-group of 256 threads: each position is covered by
// D/32 lanes, 16 bytes (32 channels) each, in both passes; lane t takes the
// positions t / (D/32) + u * 256 / (D/32), u < 9.  The whole first chunk of
// keys and then of values (576 positions at D = 128) is requested at entry,
// with nontemporal loads (the cache is read once), so one work-group has all
// its bytes in flight at once instead of a few rows per pass iteration.
//   1. scores: per lane s_g * (q . c) + min_g * sum(q) over its 32 channels
//      (the reconstruction costs no multiply per element), summed over the
//      position's lanes with DPP; scores go to LDS;
//   2. softmax with block max / sum reductions (exp2 of log2(e)-scaled scores);
//   3. values: each lane accumulates sum_j (p_j s_jg 2^-E) c_ji for its 32
//      channels -- two positions at a time, as fp32 dot products of exact
//      fp16 code pairs with the fp16 pair {p_1 s_1 2^-E, p_2 s_2 2^-E}, 2^E
//      the power of two just above the lane's largest value scale -- and
//      sum_j p_j min_jg in fp32; 2^E acc + that sum is reduced over each
//      16-lane row with DPP row rotations, then over the 16 rows through LDS.
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

// v + v from the lane that the DPP control CTRL selects (a lane whose source
// is outside the row adds 0)
template <int CTRL>
__device__ inline float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// 16-byte load of data read once (cache codes): marked nontemporal so it
// streams through the caches
__device__ inline uint4 load_stream16(const uint4* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_attention_kernel(const uint16_t* __restrict__ q, int64_t ldq,
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

  // ---- 4-bit cache: LPP lanes per position in both passes, 16 bytes (32
  // channels, half a group) each; position j = c0 + slot + u * SLOTS ----
  constexpr int LPP4 = D / 32;
  constexpr int SLOTS4 = 256 / LPP4;
  constexpr int VPOS = 9;                 // positions per lane and chunk
  constexpr int CH = VPOS * SLOTS4;       // positions per chunk (576 at D = 128)
  const int slot4 = tid / LPP4, lq = tid % LPP4, grp = lq / 2;
  uint4 kw[VPOS], vw[VPOS];
  uint32_t kmeta[VPOS], vmeta[VPOS];
  auto load_chunk = [&](const uint8_t* codes, const uint16_t* meta, uint4 (&w)[VPOS], uint32_t (&mt)[VPOS],
                        int c0) {
#pragma unroll
    for (int u = 0; u < VPOS; ++u) {
      const int j = c0 + slot4 + u * SLOTS4;
      if (j < len) {
        w[u] = load_stream16(reinterpret_cast<const uint4*>(codes + (row0 + j) * (D / 2)) + lq);
        mt[u] = reinterpret_cast<const uint32_t*>(meta)[(row0 + j) * G + grp];
      } else {
        w[u] = make_uint4(0, 0, 0, 0);
        mt[u] = 0;
      }
    }
  };
  // the first chunk of keys, then of values, requested before anything else
  load_chunk(kc, km, kw, kmeta, 0);
  load_chunk(vc, vm, vw, vmeta, 0);

  // this lane's 32 query channels as fp16 pairs, and their sum
  half2_t qv[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 r = *reinterpret_cast<const uint4*>(qp + lq * 32 + i * 8);
    qv[4 * i + 0] = __builtin_bit_cast(half2_t, r.x);
    qv[4 * i + 1] = __builtin_bit_cast(half2_t, r.y);
    qv[4 * i + 2] = __builtin_bit_cast(half2_t, r.z);
    qv[4 * i + 3] = __builtin_bit_cast(half2_t, r.w);
  }
  float qsum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) qsum += (float)qv[i].x + (float)qv[i].y;

  // ---- scores: s_g (q . c) + min_g sum(q) over this lane's 32 channels,
  // summed over the position's LPP lanes with DPP ----
  float lmax = -INFINITY;
  for (int c0 = 0; c0 < len; c0 += CH) {
    if (c0 > 0) load_chunk(kc, km, kw, kmeta, c0);
#pragma unroll
    for (int u = 0; u < VPOS; ++u) {
      const uint32_t w[4] = {kw[u].x, kw[u].y, kw[u].z, kw[u].w};
      float dc = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        half2_t cc[4];
        codes8_cvt(w[wd], cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) dc = __builtin_amdgcn_fdot2(cc[i], qv[wd * 4 + i], dc, false);
      }
      float sc = h2f((uint16_t)(kmeta[u] >> 16)) * dc + h2f((uint16_t)(kmeta[u] & 0xFFFF)) * qsum;
      sc = dpp_add<0xB1>(sc);                              // quad_perm [1, 0, 3, 2]: lane pairs
      if constexpr (LPP4 == 4) sc = dpp_add<0x4E>(sc);     // quad_perm [2, 3, 0, 1]: the quad
      sc *= kLog2e;
      const int j = c0 + slot4 + u * SLOTS4;
      if (j < len) {
        if (lq == 0) p[j] = sc;
        lmax = fmaxf(lmax, sc);
      }
    }
  }
  const float mx = block_max256(lmax, red);
  float lsum = 0.f;
  for (int j = tid; j < len; j += 256) {
    const float e = exp2f(p[j] - mx);
    p[j] = e;
    lsum += e;
  }
  const float inv = 1.0f / block_sum256(lsum, red);  // also orders the p[] writes before the reads below

  // ---- values: positions in pairs, sum_j (p_j s_j 2^-E) c_jk as fp32 dot
  // products of the fp16 pairs {c_1k, c_2k} and {p_1 s_1 2^-E, p_2 s_2 2^-E},
  // and sum_j p_j min_j in fp32.  2^E: the power of two just above the
  // largest value scale among this lane's positions so far (the products are
  // then at most 1 and fall below fp16's normal range only when 2^-14 below
  // the largest possible one); when a later chunk raises it, the sums so far
  // are rescaled (exactly) ----
  float acc[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.f;
  float bsum = 0.f;
  int vexp = 0;
  bool vset = false;  // a nonzero value scale seen
  for (int c0 = 0; c0 < len; c0 += CH) {
    if (c0 > 0) load_chunk(vc, vm, vw, vmeta, c0);
    float smx = 0.f;
#pragma unroll
    for (int u = 0; u < VPOS; ++u) smx = fmaxf(smx, h2f((uint16_t)(vmeta[u] >> 16)));  // unused slots hold 0
    int e = 0;
    (void)frexpf(smx, &e);  // smx = f * 2^e, f in [0.5, 1) (smx = 0: e = 0)
    if (smx > 0.f) {
      if (!vset) {
        vexp = e;
        vset = true;
      } else if (e > vexp) {
        const float r = ldexpf(1.0f, vexp - e);
#pragma unroll
        for (int k = 0; k < 32; ++k) acc[k] *= r;
        vexp = e;
      }
    }
    const float vsh = ldexpf(1.0f, -vexp);  // 1 until a nonzero scale is seen
#pragma unroll
    for (int u = 0; u < VPOS; u += 2) {
      const int j1 = c0 + slot4 + u * SLOTS4, j2 = j1 + SLOTS4;
      const bool two = u + 1 < VPOS;
      const float p1 = j1 < len ? p[j1] : 0.f;
      const float p2 = two && j2 < len ? p[j2] : 0.f;
      const uint32_t m1 = vmeta[u], m2 = two ? vmeta[u + 1] : 0u;
      const uint4 w1 = vw[u], w2 = two ? vw[u + 1] : make_uint4(0, 0, 0, 0);
      bsum += p1 * h2f((uint16_t)(m1 & 0xFFFF)) + p2 * h2f((uint16_t)(m2 & 0xFFFF));
      const half2_t a2 = {(half_t)(p1 * (h2f((uint16_t)(m1 >> 16)) * vsh)),
                          (half_t)(p2 * (h2f((uint16_t)(m2 >> 16)) * vsh))};
      const uint32_t x1[4] = {w1.x, w1.y, w1.z, w1.w}, x2[4] = {w2.x, w2.y, w2.z, w2.w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        half2_t cc[8];
        codes8_pairs(x1[wd], x2[wd], cc);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[wd * 8 + k] = __builtin_amdgcn_fdot2(cc[k], a2, acc[wd * 8 + k], false);
      }
    }
  }
  const float vsc_back = ldexpf(1.0f, vexp);  // 2^E, exact (1 when no nonzero scale)
  // sum over the slots of each 16-lane row (lanes l, l + LPP4, ... hold the
  // same channels) with row rotations, then over the 16 rows through LDS
  auto row_sum = [](float v) {
    if constexpr (LPP4 == 2) v = dpp_add<0x122>(v);  // row_ror 2
    v = dpp_add<0x124>(v);                           // row_ror 4
    return dpp_add<0x128>(v);                        // row_ror 8
  };
  float* part = smem + ((len + 3) & ~3);  // [16 rows][D]
  const int lane = tid & 63, row = (tid >> 6) * 4 + (lane >> 4);
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float v = row_sum(acc[k] * vsc_back + bsum);
    if ((lane & 15) < LPP4) part[row * D + lq * 32 + k] = v;
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) o += part[r * D + tid];
    out[(int64_t)b * ldo + (int64_t)h * D + tid] = f2h(o * inv);
  }
}

// ---- causal prefill on the matrix cores ------------------------------------
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// Work-group = 4 waves x 32 queries of one (b, h); keys in chunks of 64.
// Per chunk the work-group stages the chunk's K and V codes in LDS as exact
// fp16 integers (the fp16 cache: the stored values) and, for the 4-bit cache,
// each key's fp32 {min, scale} per group; then each wave computes
//   S^T = K^ Q^T      (v_mfma_f32_16x16x32_f16; lane owns query lane % 16)
//   online softmax    (per query, reduced over the 4 lane groups)
//   O^T += V^T P^T    (P taken straight from the S^T registers)
// 4-bit cache, without rounding the reconstructed cache to fp16:
//   scores, in log2 units: per group g, T_g = C_g Q_g^T over the group's 64
//     channels (exact products of fp16 queries and integer codes, fp32 sums);
//     the min terms sum_g min_g * sum(q_g) log2(e) on the matrix cores too,
//     from min_g (fp16) and each query's group sum times log2(e) split into
//     two fp16 parts (hi + lo: 22 significant bits), which start the score
//     accumulator; then one fp32 FMA per group, s += (scale_g log2(e)) T_g.
//     If a scaled group sum reaches 2^15 (fp16 would overflow) the
//     work-group takes all its scores 2^-e smaller (e > 0, exact) and
//     multiplies them back inside the exponent;
//   values: with the codes centred (c' = c - 8, exact in fp16) and
//     min' = min + 8 scale, per group g, O_g^T += C'_g^T P'_g^T with
//     P'_g = fp16(p * scale_g * 2^-E_g), 2^E_g the power of two just above the
//     largest value scale of group g among the work-group's keys (so P' <= 256
//     and leaves fp16's normal range only for terms far below the largest
//     one), plus sum_j p_j min'_jg in fp32; the output is
//     (2^E_g O_g + sum_j p_j min'_jg) / sum_j p_j.  The rounding of P' then
//     weighs |scale * c'| <= 8 scale, about the distance of the value from the
//     middle of its group's range.
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
  constexpr int KHALF = D / 64;    // K stored as D/64 arrays of 64 d (128-byte rows): array g = group g
  constexpr int MG = F16 ? 1 : G;  // {min, scale} arrays (unused with the fp16 cache)
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KHALF][KC * 64];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * KC];
  __shared__ __attribute__((aligned(16))) float ksc_lds[MG][KC], vmin_lds[MG][KC], vsc_lds[MG][KC];
  // each key's {min_g, min_g} fp16 pairs, g = 0, 1 (the A operand of the min-term product)
  __shared__ __attribute__((aligned(16))) uint32_t kmin2_lds[F16 ? 1 : KC][2];
  __shared__ float red[4][G + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  // Work-group order: the hardware deals consecutive work-groups to the 8
  // XCDs in turn, and a query block's work grows with its index (causal), so
  // the index is taken from the high part of the linear id -- every XCD gets
  // an equal share of every query block -- longest blocks first.
  // (1-D grid of query blocks x sequences x heads.)
  const int nqb = (T + 127) / 128, nbh = (int)(gridDim.x / nqb);
  const int lin = (int)blockIdx.x;
  const int qblk = nqb - 1 - lin / nbh;
  const int bh = lin % nbh, b = bh / H, h = bh % H;
  const int t0 = qblk * 128 + wave * 32;           // first query of this wave
  const int64_t row0 = ((b0 + b) * H + h) * cap;   // first cache row of this (b, h)
  const int64_t nkeys = pos + min(T, qblk * 128 + 128);

  // Q^T operand: lane (query l16 of q-block qb, d slice kd, chunk g4)
  half8_t qf[2][NKD];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = min(t0 + qb * 16 + l16, T - 1);
    const uint16_t* qp = q + ((int64_t)b * T + t) * ldq + (int64_t)h * D;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[qb][kd] = *reinterpret_cast<const half8_t*>(qp + kd * 32 + g4 * 8);
  }
  // 4-bit cache: sum of each group's query channels (query l16 of block qb)
  float qsum[2][G];
  // and 2^-E_g per value group (in LDS: read at staging and at the end);
  // sgrp = {2^-e, 2^e}, the work-group's score scaling (1 unless a query's
  // scaled group sum would overflow fp16)
  __shared__ float vmul[G], sgrp[2];
  constexpr float kL2e = 1.4426950408889634f;
  // B operand of the min-term product (16x16x16: k = 4 * lane group + i):
  // {hi, lo} of sum(q_g) log2(e) 2^-e for g = 0, 1 in lane group 0, zeros elsewhere
  half4_t qminb[2];
  float spow = 1.f;  // 2^e
  if constexpr (!F16) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sq = 0.f;
#pragma unroll
        for (int kd = 2 * g; kd < 2 * g + 2; ++kd)
#pragma unroll
          for (int e = 0; e < 8; ++e) sq += (float)qf[qb][kd][e];
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        qsum[qb][g] = sq * kL2e;
      }
    float qa = 0.f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < G; ++g) qa = fmaxf(qa, fabsf(qsum[qb][g]));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) qa = fmaxf(qa, __shfl_xor(qa, o));
    float smax[G];
#pragma unroll
    for (int g = 0; g < G; ++g) smax[g] = 0.f;
    for (int64_t j = tid; j < nkeys; j += 256)
#pragma unroll
      for (int g = 0; g < G; ++g) smax[g] = fmaxf(smax[g], h2f(vm[((row0 + j) * G + g) * 2 + 1]));
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) smax[g] = fmaxf(smax[g], __shfl_xor(smax[g], o));
      if (lane == 0) red[wave][g] = smax[g];
    }
    if (lane == 0) red[wave][G] = qa;
    __syncthreads();
    if (tid < G) {
      const int g = tid;
      const float m = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
      int e = 0;
      (void)frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1) (m = 0: e = 0)
      vmul[g] = m > 0.f ? ldexpf(1.0f, -e) : 1.0f;
      if (g == 0) {
        // smallest e >= 0 with every |sum(q_g) log2(e)| 2^-e < 2^15 (fp16 hi part finite)
        const float qm = fmaxf(fmaxf(red[0][G], red[1][G]), fmaxf(red[2][G], red[3][G]));
        int eq = 0;
        (void)frexpf(qm, &eq);  // qm < 2^eq
        const int es = eq > 15 ? eq - 15 : 0;
        sgrp[0] = ldexpf(1.0f, -es);
        sgrp[1] = ldexpf(1.0f, es);
      }
    }
    __syncthreads();
    const float sdown = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sgrp[0])));
    spow = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sgrp[1])));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      half4_t bq = {};
      if (g4 == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float v = qsum[qb][g] * sdown;  // exact (a power of two)
          const half_t hi = (half_t)v;
          bq[2 * g] = hi;
          bq[2 * g + 1] = (half_t)(v - (float)hi);  // v - hi exact in fp32
        }
      }
      qminb[qb] = bq;
    }
  }
  float4_t oacc[NDB][2];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) oacc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  float msum[2][G];  // this lane's share of sum_j p_j min_jg (4-bit cache)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g = 0; g < G; ++g) msum[qb][g] = 0.f;

  // Staging: every thread stages part of K and part of V of each chunk.
  //   K: key tid / 4, channels (tid % 4) * D/4 .. + D/4 - 1 (D/32 code words);
  //   V: channels 8 * (tid / 16) .. + 7 of the 4 positions of quad tid % 16
  //      (two quads make one 8-position storage chunk in slice order);
  //   {min, scale}: thread t < 64 G, key t % 64, group t / 64, K and V.
  // 4-bit cache: the raw codes and {min, scale} of the next chunk are loaded
  // into registers before the current chunk's products, so their latency
  // hides behind them; they are converted and stored at the next chunk's
  // start.
  constexpr int KW = D / 32;  // K code words (8 channels each) per thread
  const int kkey = tid >> 2, kq = tid & 3;
  const int vdc = tid >> 4, vpq = tid & 15;
  const int vpc = vpq >> 1, vhalf = vpq & 1;  // storage chunk, its first or second 4 positions
  const bool vact = vdc < D / 8;
  const int mkey = tid % KC, mg = tid / KC;
  const bool mact = !F16 && tid < KC * G;
  auto vkey = [&](int jj) { return (vpc >> 2) * 32 + vhalf * 16 + 4 * (vpc & 3) + jj; };
  uint32_t rk[KW], rv[4], rkm = 0, rvm = 0;
  auto load_raw = [&](int64_t k0) {
    if constexpr (!F16) {
      const int64_t j = min(k0 + kkey, nkeys - 1);
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(kc + (row0 + j) * (D / 2)) + kq * KW;
#pragma unroll
      for (int w = 0; w < KW; ++w) rk[w] = cw[w];
      if (vact) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t jv = min(k0 + vkey(jj), nkeys - 1);
          rv[jj] = reinterpret_cast<const uint32_t*>(vc + (row0 + jv) * (D / 2))[vdc];
        }
      }
      if (mact) {
        const int64_t jm = min(k0 + mkey, nkeys - 1);
        rkm = reinterpret_cast<const uint32_t*>(km)[(row0 + jm) * G + mg];
        rvm = reinterpret_cast<const uint32_t*>(vm)[(row0 + jm) * G + mg];
      }
    }
  };
  auto code_words = [](uint32_t w) {  // 8 codes -> 4 exact fp16 pairs, as one 16-byte word
    half2_t c[4];
    codes8_cvt(w, c);
    return make_uint4(__builtin_bit_cast(uint32_t, c[0]), __builtin_bit_cast(uint32_t, c[1]),
                      __builtin_bit_cast(uint32_t, c[2]), __builtin_bit_cast(uint32_t, c[3]));
  };
  auto code_words_centered = [](uint32_t w) {  // 8 codes -> 4 exact fp16 pairs of c - 8
    half2_t c[4];
    codes8_cvt(w, c);
    const half2_t eight = {(half_t)8.0f, (half_t)8.0f};
    return make_uint4(__builtin_bit_cast(uint32_t, c[0] - eight), __builtin_bit_cast(uint32_t, c[1] - eight),
                      __builtin_bit_cast(uint32_t, c[2] - eight), __builtin_bit_cast(uint32_t, c[3] - eight));
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
        if constexpr (F16)
          *reinterpret_cast<uint4*>(&k_lds[arr][at]) = *reinterpret_cast<const uint4*>(k16 + (row0 + j) * D + d0);
        else
          *reinterpret_cast<uint4*>(&k_lds[arr][at]) = code_words(rk[w]);
      }
    }
    // ---- stage V, transposed: [d][positions in slice order] ----
    if (vact) {
      uint32_t x[4][4];  // [position][channel pair]
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint4 r4;
        if constexpr (F16) {
          const int64_t jv = min(k0 + vkey(jj), nkeys - 1);
          r4 = *reinterpret_cast<const uint4*>(v16 + (row0 + jv) * D + vdc * 8);
        } else {
          r4 = code_words_centered(rv[jj]);
        }
        x[jj][0] = r4.x, x[jj][1] = r4.y, x[jj][2] = r4.z, x[jj][3] = r4.w;
      }
      // channel i: its 4 positions as 8 bytes, the first or second half of a 16-byte chunk
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = vdc * 8 + i;
        const int at = d * KC + ((vpc ^ (d & 7)) * 8) + vhalf * 4;
        auto pick = [&](int pp) {  // low halves (even channel) or high (odd)
          const uint32_t a = x[2 * pp][i >> 1], c2 = x[2 * pp + 1][i >> 1];
          return (i & 1) ? ((a >> 16) | (c2 & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c2 << 16));
        };
        *reinterpret_cast<uint2*>(&v_lds[at]) = make_uint2(pick(0), pick(1));
      }
    }
    // ---- stage {min, scale} as fp32; value scales times 2^-E_g ----
    if constexpr (!F16) {
      if (mact) {
        const float vmg = vmul[mg];
        kmin2_lds[mkey][mg] = (rkm & 0xFFFFu) * 0x00010001u;  // {min, min}
        if (G == 1) kmin2_lds[mkey][1] = 0u;
        ksc_lds[mg][mkey] = h2f((uint16_t)(rkm >> 16)) * kL2e * sgrp[0];
        const float vsf = h2f((uint16_t)(rvm >> 16));
        vmin_lds[mg][mkey] = h2f((uint16_t)(rvm & 0xFFFF)) + 8.0f * vsf;  // min + 8 s: the centre of the codes
        vsc_lds[mg][mkey] = vsf * vmg;  // exact: a power of two
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
      const int key = kb * 16 + l16;
      if constexpr (F16) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
          const int arr = kd / 2, chunk = (kd % 2) * 4 + g4;
          const half8_t kf = *reinterpret_cast<const half8_t*>(&k_lds[arr][key * 64 + ((chunk ^ (key & 7)) * 8)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[qb][kd], sacc[kb][qb], 0, 0, 0);
        }
      } else {
        // min terms first (key kb*16 + l16 in lane group 0), then group by
        // group: t = codes . q over the group's 64 channels and
        // s += scale * t for keys kb*16 + 4*g4 + r of this lane
        const int kbase = kb * 16 + 4 * g4;
        {
          // A: {min_0, min_0, min_1, min_1} of key kb*16 + l16 in every lane
          // group (B is zero outside lane group 0)
          const half4_t amin = __builtin_bit_cast(half4_t, *reinterpret_cast<const uint2*>(&kmin2_lds[key][0]));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x16f16(amin, qminb[qb], (float4_t){0.f, 0.f, 0.f, 0.f},
                                                                0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float4_t tg[2] = {(float4_t){0.f, 0.f, 0.f, 0.f}, (float4_t){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int kd = 2 * g; kd < 2 * g + 2; ++kd) {
            const int chunk = (kd % 2) * 4 + g4;
            const half8_t kf = *reinterpret_cast<const half8_t*>(&k_lds[g][key * 64 + ((chunk ^ (key & 7)) * 8)]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) tg[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[qb][kd], tg[qb], 0, 0, 0);
          }
          const float4 sc = *reinterpret_cast<const float4*>(&ksc_lds[g][kbase]);
          const float scr[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[kb][qb][r] = fmaf(scr[r], tg[qb][r], sacc[kb][qb][r]);
        }
        // the scores of this key block are formed here: the empty asm keeps
        // the compiler from sinking the combination into the softmax (which
        // would hold every block's products and {min, scale} at once)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) asm volatile("" : "+v"(sacc[kb][qb]));
      }
    }
    // ---- online softmax per query (lane l16 of each query block) ----
    // The exponent base m of a query moves only when its running maximum
    // exceeds m by more than 8 (log2 units): p = 2^(s - m) <= 256 stays well
    // inside fp16, the result is unchanged mathematically (the sum l uses the
    // same base), and the rescale of O is skipped in most chunks (a
    // wave-uniform branch).  Chunks wholly below the wave's first query and
    // inside the keys need no mask.
    // The causal mask, on chunks that cross this wave's diagonal (a
    // wave-uniform branch): key kpos = k0 + 16 kb + 4 g4 + r is kept for query
    // qpos = pos + t0 + 16 qb + l16 iff 16 kb + r - 16 qb <= dq, one compare
    // with a constant per score.  Keys at or past nkeys always fail it for a
    // query that is stored (qpos < nkeys); rows past T are never stored.
    if (k0 + KC - 1 > pos + t0) {
      const int dq = (int)(pos + t0 - k0) + l16 - 4 * g4;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[kb][qb][r] = 16 * kb + r - 16 * qb <= dq ? sacc[kb][qb][r] : -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = F16 ? sacc[kb][qb][r] * kL2e : sacc[kb][qb][r];  // 4-bit: already log2 units, 2^-e
          sacc[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= spow;  // exact
      if (__any(mx > mrun[qb] + 8.f)) {
        const float mnew = mx > mrun[qb] + 8.f ? mx : mrun[qb];
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun[qb] - mnew);
        lrun[qb] *= alpha;
        mrun[qb] = mnew;
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[i][qb] *= alpha;
#pragma unroll
        for (int g = 0; g < G; ++g) msum[qb][g] *= alpha;
      }
      const float mb = mrun[qb] == -INFINITY ? 0.f : mrun[qb];  // a row with no key yet: every p is 0
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][r], spow, -mb));
          sacc[kb][qb][r] = e;
          sum += e;
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      lrun[qb] += sum;
    }
    // ---- O^T += V^T P^T ----
    // lane's keys of slice sl: e < 4 -> block 2 sl, e >= 4 -> block 2 sl + 1 (key kb*16 + 4*g4 + r)
    if constexpr (F16) {
      half8_t pf[2][2];  // [query block][32-wide key slice], B operand of O^T
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pf[qb][sl][r] = (half_t)sacc[2 * sl][qb][r];
            pf[qb][sl][4 + r] = (half_t)sacc[2 * sl + 1][qb][r];
          }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + l16;
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int chunk = sl * 4 + g4;
          const half8_t vf = *reinterpret_cast<const half8_t*>(&v_lds[d * KC + ((chunk ^ (d & 7)) * 8)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[qb][sl], oacc[db][qb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // P'_g = fp16(p * scale * 2^-E_g), one 32-key slice at a time
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          half8_t ph[2];
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const int kb = 2 * sl + kh, kbase = kb * 16 + 4 * g4;
            const float4 vs = *reinterpret_cast<const float4*>(&vsc_lds[g][kbase]);
            const float4 vn = *reinterpret_cast<const float4*>(&vmin_lds[g][kbase]);
            const float vsr[4] = {vs.x, vs.y, vs.z, vs.w}, vnr[4] = {vn.x, vn.y, vn.z, vn.w};
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float pv = sacc[kb][qb][r];
                ph[qb][kh * 4 + r] = (half_t)fmaf(pv, vsr[r], 0.f);  // one v_fma_mix per value
                msum[qb][g] += pv * vnr[r];
              }
          }
          __builtin_amdgcn_sched_barrier(0);  // one slice's P' at a time
          const int chunk = sl * 4 + g4;
#pragma unroll
          for (int db = 4 * g; db < 4 * g + 4; ++db) {
            const int d = db * 16 + l16;
            const half8_t vf = *reinterpret_cast<const half8_t*>(&v_lds[d * KC + ((chunk ^ (d & 7)) * 8)]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph[qb], oacc[db][qb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  // ---- normalise and store: lane holds channels db*16 + 4*g4 + r of its query ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mtot[G], scale[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = msum[qb][g];
      m += __shfl_xor(m, 16);
      m += __shfl_xor(m, 32);
      mtot[g] = F16 ? 0.f : m;
      scale[g] = F16 ? 1.f : 1.0f / vmul[g];  // 2^E_g, exact
    }
    const int t = t0 + qb * 16 + l16;
    if (t >= T) continue;
    const float inv = 1.0f / lrun[qb];
    uint16_t* op = out + ((int64_t)b * T + t) * ldo + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int g = db / 4;
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (oacc[db][qb][r] * scale[g] + mtot[g]) * inv;
      const uint32_t w0 = (uint32_t)f2h(o[0]) | ((uint32_t)f2h(o[1]) << 16);
      const uint32_t w1 = (uint32_t)f2h(o[2]) | ((uint32_t)f2h(o[3]) << 16);
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
  const int64_t nwg = ceil_div(T, 128) * kv->heads * B;  // query blocks x sequences x heads
  FQ_CHECK_ARG(nwg < (int64_t)1 << 31, "fq_prefill_attention: too many work-groups");
  const dim3 grid((unsigned)nwg);
  by_format(*kv, [&](auto d, auto f16) {
    prefill_attention_mfma_kernel<decltype(d)::value, decltype(f16)::value><<<grid, dim3(256), 0, st>>>(
        q, ldq, kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, kv->heads, kv->capacity, b0, (int)T, pos, out,
        ldo, kv->k16, kv->v16);
  });
  FQ_TRY(launch_check("prefill_attention_mfma_kernel"));
  if (tk >= 0) {
    const double units = (double)B * kv->heads, d = kv->head_dim, epb = kv_is_f16(*kv) ? 2.0 : 0.5625;
    const double pairs = (double)T * pos + (double)T * (T + 1) / 2.0;  // (query, key) pairs under the causal mask
    timing_end(tk, FQ_KC_PREFILL_ATTN, units * 4.0 * pairs * d, units * (4.0 * T * d + 2.0 * (pos + T) * d * epb),
               st);
  }
  return FQ_OK;
}
