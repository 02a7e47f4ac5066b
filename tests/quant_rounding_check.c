/* CPU check of the quantiser's division-free arithmetic (the GPU library's
 * quant_group):
 *  1. codes: for fp16 inputs v >= mn and a positive fp16 scale s, with
 *     d = fl32(v - mn) and r any fp32 value within one ulp of 1/s (the
 *     hardware reciprocal's accuracy: fl32(1/s) and its two neighbours),
 *         rint(fl32(d * r))   (or, within 2^-16 of a half-integer,
 *                              rint(fl32(d / s)))
 *     equals rint(fl32(d / s)), the IEEE fp32 quotient rounded half to even,
 *     clamped to [0, 15].  Every `stride`-th positive finite fp16 scale, 16
 *     minima, every fp16 v with d <= 15.6 s.
 *  2. the scale: for every `stride`-th fp32 x in [0, 131072] (every
 *     difference of two fp16 values), with c = fl32(1/15) and
 *     y0 = fl32(x * c), fl32(fma(fl32(fma(-15, y0, x)), c, y0)) equals the
 *     IEEE quotient fl32(x / 15).
 * Arguments: stride (default 1) and offset (default 0): the scales and the
 * fp32 x taken are the offset-th, (offset + stride)-th, ..., so `stride`
 * runs with offsets 0..stride-1 cover every case.
 * Prints the counts; exit status 1 on a mismatch.  Build with
 * -ffp-contract=off.  Test infrastructure: shares nothing with the GPU
 * library. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float h2f(uint16_t h) { /* exact fp16 -> fp32 */
  const uint32_t sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
  return sign ? -v : v;
}

int main(int argc, char** argv) {
  const unsigned stride = argc > 1 ? (unsigned)atoi(argv[1]) : 1;
  const unsigned offset = argc > 2 ? (unsigned)atoi(argv[2]) : 0;
  static const uint16_t mins[] = {0x0000, 0xBC00, 0xBC00 | 0x0123, 0xC500, 0x2E66, 0xA1F0, 0x1234, 0x9876,
                                  0xD000, 0x5000, 0x0400, 0x8400, 0x0001, 0x8001, 0x7BFF, 0xFBFF};
  long long checked = 0, fallback = 0, bad = 0;
  for (uint32_t sh = 1 + offset; sh < 0x7C00; sh += stride) {
    const float s = h2f((uint16_t)sh);
    const float r0 = 1.0f / s;
    for (int ri = -1; ri <= 1; ++ri) {
    const float r = ri == 0 ? r0 : nextafterf(r0, ri < 0 ? 0.0f : INFINITY);
    for (unsigned mi = 0; mi < sizeof(mins) / sizeof(mins[0]); ++mi) {
      const float mn = h2f(mins[mi]);
      for (uint32_t vh = 0; vh < 0x10000; ++vh) {
        if ((vh & 0x7C00) == 0x7C00) continue; /* inf / nan */
        const float v = h2f((uint16_t)vh);
        if (!(v >= mn)) continue;
        const float d = v - mn;
        if (d > 15.6f * s) continue;
        const float exact = fminf(fmaxf(rintf(d / s), 0.f), 15.f);
        float q = d * r;
        const int near = fabsf(q - rintf(q)) > 0.5f - 0x1p-16f;
        if (near) q = d / s;
        const float code = fminf(fmaxf(rintf(q), 0.f), 15.f);
        ++checked;
        fallback += near;
        if (code != exact) {
          if (bad < 10) printf("mismatch: s=%a r=%a mn=%a v=%a\n", s, r, mn, v);
          ++bad;
        }
      }
    }
    }
  }
  /* 2. the scale's division by 15 */
  const float c15 = 1.0f / 15.0f;
  long long checked15 = 0;
  for (uint64_t b = offset; b <= 0x48000000u; b += stride) { /* 0x48000000 = 131072.0f */
    const uint32_t bits = (uint32_t)b;
    float x;
    memcpy(&x, &bits, 4);
    const float e = x / 15.0f;
    const float y0 = x * c15;
    const float y = fmaf(fmaf(-15.0f, y0, x), c15, y0);
    ++checked15;
    if (memcmp(&e, &y, 4) != 0) {
      if (bad < 10) printf("mismatch /15: x=%a\n", x);
      ++bad;
    }
  }
  printf("checked %lld fallback %lld scales %lld mismatches %lld\n", checked, fallback, checked15, bad);
  return bad != 0;
}
