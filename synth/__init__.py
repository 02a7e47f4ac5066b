"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle.

This module holds no arithmetic of the compression method: it only produces
the fp16 weights, hidden states and token ids that the method consumes.  The
GPU library carries its own, independent implementation of the same
counter-based generator (it fills model weights in HBM); the two agree bit for
bit because every step below is exact integer arithmetic followed by exactly
two IEEE round-to-nearest-even conversions.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast Splittable
Pseudorandom Number Generators", OOPSLA 2014), used in counter form: the
64-bit output for counter i of a stream is mix64(key + (i + 1) * GAMMA), which
equals the (i+1)-th output of a SplitMix64 sequence seeded with ``key``.

Normal variates: the sum of the four 16-bit lanes of one output is an
Irwin-Hall(4) variate on 0..262140.  Centred (minus 131070) it is an exact
integer below 2**18, so its fp32 conversion is exact; it is multiplied by one
fp32 constant ``sigma / std`` (std = sqrt((65536**2 - 1) / 3), the lane-sum's
standard deviation) and rounded once to fp16.  The result has mean 0,
standard deviation sigma, and support +-3.46 sigma: a bounded stand-in for
N(0, sigma^2) with the same variance.

Token ids: Lemire's multiply-shift on the high 32 bits, ((u >> 32) * V) >> 32.

Heavy-tailed test inputs (NumPy only; the library has no counterpart):
Student's t(3), Laplace and a normal with 1-in-64 outliers, from the same
counters through float64 transforms (heavy_tailed_f16).
"""
from .gen import (GAMMA, MASK64, mix64, stream_key, raw_u64, normal_f16, normal_scale_f32,
                  token_ids, heavy_tailed_f16, STREAM, TENSOR)

__all__ = ["GAMMA", "MASK64", "mix64", "stream_key", "raw_u64", "normal_f16", "normal_scale_f32",
           "token_ids", "heavy_tailed_f16", "STREAM", "TENSOR"]
