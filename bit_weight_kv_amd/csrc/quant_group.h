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

#include <type_traits>

#include "common.h"

namespace fq {

// v: this lane's NV values (fp32 images of fp16 values, in channel order).
// packed[w]: codes of values 8w..8w+7 as nibbles (value 8w in bits 0..3).
// meta_bits: the group's fp16 min (low half) and scale (high half).
// No contraction: (x - min) / s and (max - min) / 15 round separately.
//
// The code is rint(fl32((x - min) / s)) (IEEE fp32 divide), computed without
// a divide per element: with r within one ulp of 1/s (the hardware
// reciprocal), qa = fl32((x - min) * r) differs from the correctly rounded
// quotient q by less than 2^-17 for q < 16 (relative errors of at most 2^-23
// in r and 2^-24 in the product give |qa - q_exact| < 2^-18.4, and q is within
// 2^-20 of q_exact), so wherever qa lies farther than 2^-16 from a
// half-integer both round to the same integer; a lane holding a value closer
// than that takes the exact divide for all its values.  A CPU check of the
// same fp32 operations over every fp16 scale (each reciprocal within one ulp),
// 16 minima and every fp16 value in range found no difference.
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
  // across the group's lanes (an aligned run of 4 or 8) with DPP moves:
  // swap neighbours, swap pairs within the quad, then (8 lanes) mirror the
  // two quads of the half-row, so every lane ends with the group's extremes
  static_assert(LANES == 4 || LANES == 8, "4 or 8 lanes per group");
  // (a lane whose source lane is inactive keeps its own value: neutral for min/max)
  auto dpp = [](float x, auto ctrl) {
    const int b = __builtin_bit_cast(int, x);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, decltype(ctrl)::value, 0xF, 0xF, false));
  };
  using quad_swap1 = std::integral_constant<int, 0xB1>;      // quad_perm [1, 0, 3, 2]
  using quad_swap2 = std::integral_constant<int, 0x4E>;      // quad_perm [2, 3, 0, 1]
  using half_mirror = std::integral_constant<int, 0x141>;    // row_half_mirror: lane i <-> 7 - i
  mn = fminf(mn, dpp(mn, quad_swap1{}));
  mx = fmaxf(mx, dpp(mx, quad_swap1{}));
  mn = fminf(mn, dpp(mn, quad_swap2{}));
  mx = fmaxf(mx, dpp(mx, quad_swap2{}));
  if constexpr (LANES == 8) {
    mn = fminf(mn, dpp(mn, half_mirror{}));
    mx = fmaxf(mx, dpp(mx, half_mirror{}));
  }
  if (mn == 0.0f) mn = 0.0f;  // canonical +0 minimum
  // s32 = fl32((mx - mn) / 15): the product with fl32(1/15) and one FMA
  // correction give the IEEE quotient for every fp32 difference up to 2^17
  // (checked exhaustively on the CPU)
  const float x = mx - mn;
  constexpr float c15 = 1.0f / 15.0f;
  const float y0 = x * c15;
  float s32 = __builtin_fmaf(__builtin_fmaf(-15.0f, y0, x), c15, y0);
  if (s32 == 0.0f) s32 = 0.0f;  // canonical +0 scale
  const half_t s16 = (half_t)s32;
  const float s = (float)s16;
#pragma unroll
  for (int w = 0; w < NV / 8; ++w) packed[w] = 0;
  if (s != 0.0f) {
    const float r = __builtin_amdgcn_rcpf(s);  // within one ulp of 1/s
    float c[NV];
    float far = 0.0f;  // largest distance of a quotient from its nearest integer
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float q = (v[j] - mn) * r;
      c[j] = rintf(q);
      far = fmaxf(far, fabsf(q - c[j]));
    }
    // rare: a quotient within 2^-16 of a half-integer -- this lane's values
    // take the IEEE quotient, behind a wave-uniform branch so that the
    // divides are not executed (and discarded) everywhere
    const bool near = far > 0.5f - 0x1p-16f;
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
      if (near) {
#pragma unroll
        for (int j = 0; j < NV; ++j) c[j] = rintf((v[j] - mn) / s);
      }
    }
    // clamp, then 4 codes per exact fp32 integer c0 + 16 (c1 + 16 (c2 + 16 c3))
#pragma unroll
    for (int j = 0; j < NV; j += 4) {
      float k[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) k[e] = fminf(fmaxf(c[j + e], 0.0f), 15.0f);
      const float h = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(k[3], 16.0f, k[2]), 16.0f, k[1]), 16.0f, k[0]);
      packed[j / 8] |= (uint32_t)h << (16 * ((j / 4) % 2));
    }
  }
  meta_bits = (uint32_t)f2h(mn) | ((uint32_t)__builtin_bit_cast(uint16_t, s16) << 16);
}

}  // namespace fq
