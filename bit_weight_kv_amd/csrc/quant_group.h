// Group-wise 4-bit min/max quantisation of one group of 64 values spread over
// LANES consecutive lanes (NV values per lane, NV * LANES == 64), shared by
// the quantise / append kernels and the QKV GEMM epilogue that appends K/V to
// the cache, so both produce identical codes.
//
// Method: FlexGen README (giters.com mirror), key features, "Extreme
// Compression" (weights and the attention cache in 4 bits).  Group size 64,
// min/max asymmetric range, fp16 {min, scale} metadata, IEEE fp32 arithmetic
// with round-half-to-even are this library's readings (include/fq.h).
#pragma once

#include "common.h"

namespace fq {

// v: this lane's NV values (fp32 images of fp16 values, in channel order).
// packed[w]: codes of values 8w..8w+7 as nibbles (value 8w in bits 0..3).
// meta_bits: the group's fp16 min (low half) and scale (high half).
// No contraction: (x - min) / s and (max - min) / 15 round separately.
template <int NV, int LANES>
__device__ inline void quant_group(const float (&v)[NV], uint32_t (&packed)[NV / 8], uint32_t& meta_bits) {
#pragma clang fp contract(off)
  static_assert(NV * LANES == 64 && NV % 8 == 0, "one group of 64 values");
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int j = 1; j < NV; ++j) {
    mn = fminf(mn, v[j]);
    mx = fmaxf(mx, v[j]);
  }
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (mn == 0.0f) mn = 0.0f;  // canonical +0 minimum
  float s32 = (mx - mn) / 15.0f;
  if (s32 == 0.0f) s32 = 0.0f;  // canonical +0 scale
  const half_t s16 = (half_t)s32;
  const float s = (float)s16;
#pragma unroll
  for (int w = 0; w < NV / 8; ++w) packed[w] = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float q = rintf((v[j] - mn) / s);
      q = fminf(fmaxf(q, 0.0f), 15.0f);
      packed[j / 8] |= (uint32_t)q << (4 * (j % 8));
    }
  }
  meta_bits = (uint32_t)f2h(mn) | ((uint32_t)__builtin_bit_cast(uint16_t, s16) << 16);
}

}  // namespace fq
