"""Pins of the oracle's dense operations: brute-force loops on tiny inputs,
special cases with closed forms, and special cases that reduce to library
routines (torch CPU float64)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import (quantize, dequant_f16, dequant_f64, gemm, layernorm, attention_decode,
                    attention_prefill_causal)


def _grid_exact_weight(n, k, seed=0):
    """A weight whose every group lies on its own 4-bit grid: per group mn = -m/8 and
    s = 2^-e with codes in 0..15 and both extremes present, so quantisation is lossless."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (n, k))
    codes[:, ::64] = 0
    codes[:, 1::64] = 15
    g = k // 64
    mn = -rng.integers(1, 16, (n, g)) / 8.0
    s = 2.0 ** -rng.integers(3, 7, (n, g))
    w = mn.repeat(64, 1) + codes * s.repeat(64, 1)
    return w.astype(np.float16), codes


def test_dequant_gemm_equals_textbook_gemm_on_grid_exact_weights():
    w, _ = _grid_exact_weight(48, 256)
    codes, meta = quantize(w)
    wd = dequant_f16(codes, meta)
    assert np.array_equal(wd, w)
    x = synth.normal_f16(0, synth.STREAM["aux"], (9, 256), 1.0)
    y = gemm(x, wd)
    # pure-Python triple loop in exact arithmetic (fractions are exact for binary floats)
    from fractions import Fraction
    for i in (0, 4, 8):
        for j in (0, 17, 47):
            ref = sum(Fraction(float(x[i, kk])) * Fraction(float(w[j, kk])) for kk in range(256))
            assert abs(float(ref) - y[i, j]) <= 1e-12 * max(1.0, abs(float(ref)))


def test_gemm_one_hot_rows_pick_weight_rows():
    w = synth.normal_f16(0, synth.STREAM["aux"] + 1, (32, 128), 0.02)
    codes, meta = quantize(w)
    wd = dequant_f16(codes, meta)
    b = synth.normal_f16(0, synth.STREAM["aux"] + 2, (32,), 0.02)
    x = np.zeros((3, 128), np.float16)
    x[0, 5] = 1
    x[1, 127] = 1
    x[2, 64] = 1
    y = gemm(x, wd, b)
    for r, col in enumerate((5, 127, 64)):
        assert np.array_equal(y[r], wd[:, col].astype(np.float64) + b.astype(np.float64))


def test_gemm_against_torch_float64():
    x = synth.normal_f16(0, synth.STREAM["aux"] + 3, (17, 192), 1.0)
    w = synth.normal_f16(0, synth.STREAM["aux"] + 4, (40, 192), 0.02)
    b = synth.normal_f16(0, synth.STREAM["aux"] + 5, (40,), 0.02)
    wd = dequant_f16(*quantize(w))
    ref = torch.nn.functional.linear(torch.from_numpy(x.astype(np.float64)),
                                     torch.from_numpy(wd.astype(np.float64)),
                                     torch.from_numpy(b.astype(np.float64))).numpy()
    np.testing.assert_allclose(gemm(x, wd, b), ref, rtol=1e-12, atol=1e-12)


def test_layernorm_closed_forms_and_library():
    h = 256
    g = np.ones(h, np.float16)
    b = np.zeros(h, np.float16)
    const = np.full((2, h), 3.5, np.float16)
    assert np.array_equal(layernorm(const, g, b), np.zeros((2, h)))      # x - mean = 0 -> beta
    pm = np.tile(np.array([-1.0, 1.0], np.float16), h // 2)[None]
    np.testing.assert_allclose(layernorm(pm, g, b), pm.astype(np.float64) / math.sqrt(1 + 1e-5), rtol=1e-15)
    x = synth.normal_f16(0, synth.STREAM["aux"] + 6, (5, h), 1.0)
    gg = synth.normal_f16(0, synth.STREAM["aux"] + 7, (h,), 1.0)
    bb = synth.normal_f16(0, synth.STREAM["aux"] + 8, (h,), 0.1)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (h,),
                                         torch.from_numpy(gg.astype(np.float64)),
                                         torch.from_numpy(bb.astype(np.float64)), eps=1e-5).numpy()
    np.testing.assert_allclose(layernorm(x, gg, bb), ref, rtol=1e-12, atol=1e-12)


def _rand_cache(B, H, n, d, seed):
    k = synth.normal_f16(seed, synth.STREAM["aux"] + 10, (B, H, n, d), 1.0)
    v = synth.normal_f16(seed, synth.STREAM["aux"] + 11, (B, H, n, d), 1.0)
    return dequant_f64(*quantize(k)), dequant_f64(*quantize(v))


def test_attention_single_token_returns_value():
    kh, vh = _rand_cache(2, 3, 1, 128, 0)
    q = synth.normal_f16(0, synth.STREAM["aux"] + 12, (2, 3, 128), 1.0)
    assert np.array_equal(attention_decode(q, kh, vh), vh[:, :, 0])


def test_attention_equal_keys_give_mean_value():
    kh, vh = _rand_cache(1, 2, 7, 64, 1)
    kh[:] = kh[:, :, :1]
    q = synth.normal_f16(1, synth.STREAM["aux"] + 12, (1, 2, 64), 1.0)
    np.testing.assert_allclose(attention_decode(q, kh, vh), vh.mean(2), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(attention_decode(np.zeros_like(q), _rand_cache(1, 2, 7, 64, 2)[0], vh),
                               vh.mean(2), rtol=1e-13, atol=1e-13)


def test_attention_dominant_key():
    kh, vh = _rand_cache(1, 1, 6, 64, 3)
    q = np.zeros((1, 1, 64))
    q[0, 0, 0] = 1.0
    kh[0, 0, :, 0] = 0.0
    kh[0, 0, 4, 0] = 60.0           # score 60 against 0: weight 1 - 5e-26
    np.testing.assert_allclose(attention_decode(q, kh, vh)[0, 0], vh[0, 0, 4], rtol=0, atol=1e-20)


def test_attention_brute_force_loops():
    kh, vh = _rand_cache(1, 1, 8, 64, 4)
    q = synth.normal_f16(4, synth.STREAM["aux"] + 13, (1, 1, 64), 1.0).astype(np.float64) / 8
    for n in range(1, 9):
        s = [sum(q[0, 0, i] * kh[0, 0, j, i] for i in range(64)) for j in range(n)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        o = [sum(e[j] / z * vh[0, 0, j, i] for j in range(n)) for i in range(64)]
        np.testing.assert_allclose(attention_decode(q, kh[:, :, :n], vh[:, :, :n])[0, 0], o,
                                   rtol=1e-12, atol=1e-13)


def test_prefill_causal_against_torch_sdpa():
    kh, vh = _rand_cache(2, 2, 9, 64, 5)
    q = synth.normal_f16(5, synth.STREAM["aux"] + 14, (2, 2, 9, 64), 1.0).astype(np.float64) / 8
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(kh), torch.from_numpy(vh), is_causal=True, scale=1.0).numpy()
    np.testing.assert_allclose(attention_prefill_causal(q, kh, vh), ref, rtol=1e-12, atol=1e-12)
    # the last causal row equals a decode over all keys
    np.testing.assert_allclose(attention_prefill_causal(q, kh, vh)[:, :, -1],
                               attention_decode(q[:, :, -1], kh, vh), rtol=1e-13, atol=1e-13)
