"""Decode attention (one query per sequence) and causal prefill attention over
the packed 4-bit cache and over the fp16 cache, against the oracle's float64
softmax attention on the same cache contents.  The GPU fills its cache with its
own append (quantise-on-append for the 4-bit cache) from the same fp16 K/V
(bit-exactness of that step is tested separately)."""
import numpy as np
import pytest
import torch

import synth
import oracle
from tests._util import dev, host, assert_close, log

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")


def _cache(B, H, d, n, cap, seed, b_off=0, fmt="q4", v_sigma=1.0, k_sigma=1.0):
    """fp16 K/V [B, n, H*d] from the generator -> GPU cache (appended) and the
    oracle's reading of the same cache (fmt "q4": 4-bit, "f16": fp16)."""
    h = H * d
    k = synth.normal_f16(seed, synth.STREAM["aux"] + 20, (B * n, h), k_sigma)
    v = synth.normal_f16(seed, synth.STREAM["aux"] + 21, (B * n, h), v_sigma)
    if fmt == "q4":
        kc = torch.zeros((B + b_off, H, cap, d // 2), dtype=torch.uint8, device="cuda:0")
        km = torch.zeros((B + b_off, H, cap, d // 64, 2), dtype=torch.float16, device="cuda:0")
        vc, vm = torch.zeros_like(kc), torch.zeros_like(km)
        view, keep = fq.kv_layer_view(kc, km, vc, vm), (kc, km, vc, vm)
    else:
        k16 = torch.zeros((B + b_off, H, cap, d), dtype=torch.float16, device="cuda:0")
        v16 = torch.zeros_like(k16)
        view, keep = fq.kv_layer_view_f16(k16, v16), (k16, v16)
    kd, vd = dev(k), dev(v)
    fq.fq_kv_append(view, kd, vd, h, b_off, B, n, 0)
    torch.cuda.synchronize()
    to4 = lambda a: np.ascontiguousarray(a.reshape(B, n, H, d).transpose(0, 2, 1, 3))
    if fmt == "q4":
        kh = oracle.dequant_f64(*oracle.quantize(to4(k)))
        vh = oracle.dequant_f64(*oracle.quantize(to4(v)))
    else:
        kh, vh = to4(k).astype(np.float64), to4(v).astype(np.float64)
    return view, keep, kh, vh


@pytest.mark.parametrize("fmt", ["q4", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("length", [1, 2, 63, 64, 65, 300, 543])
def test_decode_attention(d, length, fmt):
    B, H = 3, 4
    log(f"decode attention {fmt} d={d} len={length}")
    view, keep, kh, vh = _cache(B, H, d, length, length + 3, seed=d + length, b_off=1, fmt=fmt)
    q = (synth.normal_f16(0, synth.STREAM["aux"] + 22, (B, H * d), 1.0).astype(np.float32)
         * d ** -0.5).astype(np.float16)
    out = torch.empty((B, H * d), dtype=torch.float16, device="cuda:0")
    fq.fq_decode_attention(dev(q), view, 1, B, length, out)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(q.reshape(B, H, d), kh, vh).reshape(B, H * d)
    assert_close(host(out), ref, rel=2e-3, abs_=4e-3, what=f"decode {fmt} d={d} len={length}")


@pytest.mark.parametrize("fmt", ["q4", "f16"])
def test_decode_attention_long_and_peaked(fmt):
    """A long cache (4000 positions) and a query aligned with one key (peaked softmax)."""
    B, H, d, n = 2, 2, 128, 4000
    view, keep, kh, vh = _cache(B, H, d, n, n, seed=9, fmt=fmt)
    q = np.zeros((B, H, d), np.float16)
    q[:, :, :] = (kh[:, :, 1234, :] * 0.3).astype(np.float16)
    out = torch.empty((B, H * d), dtype=torch.float16, device="cuda:0")
    fq.fq_decode_attention(dev(q.reshape(B, H * d)), view, 0, B, n, out)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(q, kh, vh).reshape(B, H * d)
    assert_close(host(out), ref, rel=2e-3, abs_=4e-3, what="long/peaked")


@pytest.mark.parametrize("fmt", ["q4", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,pos", [(1, 0), (5, 0), (64, 0), (65, 0), (130, 0), (9, 7), (300, 40), (600, 23)])
def test_prefill_attention_causal(d, T, pos, fmt):
    """Causal attention of T new tokens after pos cached ones against the
    oracle's attention per query; (600, 23): five 128-query blocks per (b, h),
    the last one ragged, dealt over the XCDs longest first."""
    B, H = 2, 3
    kernel = "mfma"
    log(f"prefill attention {fmt} d={d} T={T} pos={pos}")
    n = pos + T
    view, keep, kh, vh = _cache(B, H, d, n, n + 1, seed=T + pos, fmt=fmt)
    q = (synth.normal_f16(1, synth.STREAM["aux"] + 23, (B * T, H * d), 1.0).astype(np.float32)
         * d ** -0.5).astype(np.float16)
    out = torch.empty((B * T, H * d), dtype=torch.float16, device="cuda:0")
    fq.fq_prefill_attention(dev(q), view, 0, B, T, pos, out)
    torch.cuda.synchronize()
    q4 = q.reshape(B, T, H, d).transpose(0, 2, 1, 3).astype(np.float64)
    ref = np.empty((B, H, T, d))
    for t in range(T):
        ref[:, :, t] = oracle.attention_decode(q4[:, :, t], kh[:, :, :pos + t + 1], vh[:, :, :pos + t + 1])
    ref = ref.transpose(0, 2, 1, 3).reshape(B * T, H * d)
    r, m = assert_close(host(out), ref, rel=2e-3, abs_=4e-3, what=f"prefill {kernel} {fmt} d={d} T={T} pos={pos}")
    log(f"prefill {kernel} {fmt} d={d} T={T} pos={pos}: rel_l2 {r:.2e} max_abs {m:.2e}")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_attention_large_query_sums(d):
    """Queries whose channel sums over a quantisation group exceed what fp16
    holds once scaled by log2(e) (every channel 400 + N(0, 20): about 25600 per
    group, 36900 in log2 units): the 4-bit prefill kernel then takes all its
    scores 2^-1 smaller for the min-term product and restores them in the
    exponent.  Keys of small spread (sigma 1e-3) keep the softmax from
    collapsing onto one key: the min terms (min_g times the group sums) are
    the large part of every score.  Held to the same bounds as the other
    prefill cases against the oracle's float64 attention."""
    B, H, T, pos = 2, 3, 130, 20
    n = pos + T
    view, keep, kh, vh = _cache(B, H, d, n, n + 1, seed=77 + d, fmt="q4", k_sigma=1e-3)
    q = (400.0 + synth.normal_f16(2, synth.STREAM["aux"] + 24, (B * T, H * d), 20.0).astype(np.float32)).astype(
        np.float16)
    qs = q.astype(np.float64).reshape(B * T, H, d // 64, 64).sum(-1) * 1.4426950408889634
    assert qs.min() > 2.0 ** 15  # the rescaled path
    out = torch.empty((B * T, H * d), dtype=torch.float16, device="cuda:0")
    fq.fq_prefill_attention(dev(q), view, 0, B, T, pos, out)
    torch.cuda.synchronize()
    q4 = q.reshape(B, T, H, d).transpose(0, 2, 1, 3).astype(np.float64)
    ref = np.empty((B, H, T, d))
    for t in range(T):
        ref[:, :, t] = oracle.attention_decode(q4[:, :, t], kh[:, :, :pos + t + 1], vh[:, :, :pos + t + 1])
    ref = ref.transpose(0, 2, 1, 3).reshape(B * T, H * d)
    r, m = assert_close(host(out), ref, rel=2e-3, abs_=4e-3, what=f"prefill large query sums d={d}")
    log(f"prefill large query sums d={d}: rel_l2 {r:.2e} max_abs {m:.2e}")


@pytest.mark.parametrize("v_sigma", [2.0 ** -8, 64.0])
def test_attention_value_scale_range(v_sigma):
    """Values far below and above unit size: the value pass rounds p * scale
    (times a power of two chosen from the largest scale) to fp16; the outputs
    keep the same relative accuracy as at unit size, in decode and prefill,
    over a cache long enough to span several chunks of the decode kernel."""
    B, H, d = 2, 3, 128
    n = 1300
    log(f"value scale range sigma={v_sigma}")
    view, keep, kh, vh = _cache(B, H, d, n, n, seed=77, v_sigma=v_sigma)
    q = (synth.normal_f16(0, synth.STREAM["aux"] + 22, (B, H * d), 1.0).astype(np.float32)
         * d ** -0.5).astype(np.float16)
    out = torch.empty((B, H * d), dtype=torch.float16, device="cuda:0")
    fq.fq_decode_attention(dev(q), view, 0, B, n, out)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(q.reshape(B, H, d), kh, vh).reshape(B, H * d)
    assert_close(host(out), ref, rel=2e-3, abs_=4e-3 * v_sigma, what=f"decode sigma={v_sigma}")
    T, pos = 200, n - 200
    qp = (synth.normal_f16(1, synth.STREAM["aux"] + 23, (B * T, H * d), 1.0).astype(np.float32)
          * d ** -0.5).astype(np.float16)
    outp = torch.empty((B * T, H * d), dtype=torch.float16, device="cuda:0")
    fq.fq_prefill_attention(dev(qp), view, 0, B, T, pos, outp)
    torch.cuda.synchronize()
    q4 = qp.reshape(B, T, H, d).transpose(0, 2, 1, 3).astype(np.float64)
    refp = np.empty((B, H, T, d))
    for t in range(T):
        refp[:, :, t] = oracle.attention_decode(q4[:, :, t], kh[:, :, :pos + t + 1], vh[:, :, :pos + t + 1])
    refp = refp.transpose(0, 2, 1, 3).reshape(B * T, H * d)
    assert_close(host(outp), refp, rel=2e-3, abs_=4e-3 * v_sigma, what=f"prefill sigma={v_sigma}")


@pytest.mark.parametrize("d", [64, 128])
def test_attention_value_scale_growing_along_the_cache(d):
    """Value magnitudes that grow along the cache (x 2^-6 for the first 600
    positions, x 4 after): the decode kernel's per-lane power-of-two value scale
    is raised by a later chunk of positions and the sums so far are rescaled;
    the prefill kernel takes its power of two from every key it reads.  Both
    against the oracle's float64 attention over the same cache."""
    B, H, n = 2, 3, 1500
    h = H * d
    k = synth.normal_f16(3, synth.STREAM["aux"] + 24, (B * n, h), 1.0)
    v = synth.normal_f16(3, synth.STREAM["aux"] + 25, (B * n, h), 1.0).astype(np.float32)
    grow = np.where(np.arange(n) < 600, 2.0 ** -6, 4.0).astype(np.float32)
    v = (v.reshape(B, n, h) * grow[None, :, None]).reshape(B * n, h).astype(np.float16)
    kc = torch.zeros((B, H, n, d // 2), dtype=torch.uint8, device="cuda:0")
    km = torch.zeros((B, H, n, d // 64, 2), dtype=torch.float16, device="cuda:0")
    vc, vm = torch.zeros_like(kc), torch.zeros_like(km)
    view = fq.kv_layer_view(kc, km, vc, vm)
    fq.fq_kv_append(view, dev(k), dev(v), h, 0, B, n, 0)
    torch.cuda.synchronize()
    to4 = lambda a: np.ascontiguousarray(a.reshape(B, n, H, d).transpose(0, 2, 1, 3))
    kh = oracle.dequant_f64(*oracle.quantize(to4(k)))
    vh = oracle.dequant_f64(*oracle.quantize(to4(v)))
    q = (synth.normal_f16(0, synth.STREAM["aux"] + 26, (B, h), 1.0).astype(np.float32) * d ** -0.5).astype(np.float16)
    out = torch.empty((B, h), dtype=torch.float16, device="cuda:0")
    fq.fq_decode_attention(dev(q), view, 0, B, n, out)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(q.reshape(B, H, d), kh, vh).reshape(B, h)
    assert_close(host(out), ref, rel=2e-3, abs_=1.6e-2, what=f"decode d={d} growing values")
    T, pos = 130, n - 130
    qp = (synth.normal_f16(1, synth.STREAM["aux"] + 27, (B * T, h), 1.0).astype(np.float32)
          * d ** -0.5).astype(np.float16)
    outp = torch.empty((B * T, h), dtype=torch.float16, device="cuda:0")
    fq.fq_prefill_attention(dev(qp), view, 0, B, T, pos, outp)
    torch.cuda.synchronize()
    q4 = qp.reshape(B, T, H, d).transpose(0, 2, 1, 3).astype(np.float64)
    refp = np.empty((B, H, T, d))
    for t in range(T):
        refp[:, :, t] = oracle.attention_decode(q4[:, :, t], kh[:, :, :pos + t + 1], vh[:, :, :pos + t + 1])
    refp = refp.transpose(0, 2, 1, 3).reshape(B * T, h)
    assert_close(host(outp), refp, rel=2e-3, abs_=1.6e-2, what=f"prefill d={d} growing values")


def test_decode_full_size_sampled():
    """OPT-175B shape at decode: batch 144, 96 heads x 128, 543 cached positions;
    the cache is filled for all sequences, sampled (b, h) pairs are checked."""
    B, H, d, n = 144, 96, 128, 543
    h = H * d
    log("decode attention full-size")
    kc = torch.empty((B, H, n, d // 2), dtype=torch.uint8, device="cuda:0")
    km = torch.empty((B, H, n, d // 64, 2), dtype=torch.float16, device="cuda:0")
    vc, vm = torch.empty_like(kc), torch.empty_like(km)
    view = fq.kv_layer_view(kc, km, vc, vm)
    chunk = 16
    kbuf = torch.empty((chunk * n, h), dtype=torch.float16, device="cuda:0")
    vbuf = torch.empty_like(kbuf)
    for b0 in range(0, B, chunk):
        fq.fq_synth_normal_f16(kbuf, 5, synth.STREAM["aux"] + 30, 1.0, first=b0 * n * h)
        fq.fq_synth_normal_f16(vbuf, 5, synth.STREAM["aux"] + 31, 1.0, first=b0 * n * h)
        fq.fq_kv_append(view, kbuf, vbuf, h, b0, chunk, n, 0)
    qd = torch.empty((B, h), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(qd, 5, synth.STREAM["aux"] + 32, 1.0 / d ** 0.5)
    out = torch.empty((B, h), dtype=torch.float16, device="cuda:0")
    fq.fq_decode_attention(qd, view, 0, B, n, out)
    torch.cuda.synchronize()
    for b, hh in ((0, 0), (77, 41), (143, 95)):
        base = (b * n + np.arange(n))[:, None] * h + hh * d + np.arange(d)[None]
        k = synth.normal_f16(5, synth.STREAM["aux"] + 30, sigma=1.0, index=base.astype(np.uint64).ravel()).reshape(n, d)
        v = synth.normal_f16(5, synth.STREAM["aux"] + 31, sigma=1.0, index=base.astype(np.uint64).ravel()).reshape(n, d)
        qi = (b * h + hh * d + np.arange(d)).astype(np.uint64)
        q = synth.normal_f16(5, synth.STREAM["aux"] + 32, sigma=1.0 / d ** 0.5, index=qi)
        kh = oracle.dequant_f64(*oracle.quantize(k))[None, None]
        vh = oracle.dequant_f64(*oracle.quantize(v))[None, None]
        ref = oracle.attention_decode(q[None, None], kh, vh)[0, 0]
        got = host(out[b, hh * d:(hh + 1) * d])
        assert_close(got, ref, rel=2e-3, abs_=4e-3, what=f"full-size b={b} h={hh}")


def test_prefill_full_size_sampled():
    """OPT-175B shape at prefill: 144 sequences x 96 heads x 128, a 512-token
    prompt attended causally over its 4-bit cache in the launch the prompt pass
    makes; sampled (b, h) pairs checked at every query position."""
    B, H, d, T = 144, 96, 128, 512
    h = H * d
    log("prefill attention full-size")
    kc = torch.empty((B, H, T, d // 2), dtype=torch.uint8, device="cuda:0")
    km = torch.empty((B, H, T, d // 64, 2), dtype=torch.float16, device="cuda:0")
    vc, vm = torch.empty_like(kc), torch.empty_like(km)
    view = fq.kv_layer_view(kc, km, vc, vm)
    chunk = 16
    kbuf = torch.empty((chunk * T, h), dtype=torch.float16, device="cuda:0")
    vbuf = torch.empty_like(kbuf)
    for b0 in range(0, B, chunk):
        fq.fq_synth_normal_f16(kbuf, 6, synth.STREAM["aux"] + 33, 1.0, first=b0 * T * h)
        fq.fq_synth_normal_f16(vbuf, 6, synth.STREAM["aux"] + 34, 1.0, first=b0 * T * h)
        fq.fq_kv_append(view, kbuf, vbuf, h, b0, chunk, T, 0)
    del kbuf, vbuf
    qd = torch.empty((B * T, h), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(qd, 6, synth.STREAM["aux"] + 35, 1.0 / d ** 0.5)
    out = torch.empty((B * T, h), dtype=torch.float16, device="cuda:0")
    fq.fq_prefill_attention(qd, view, 0, B, T, 0, out)
    torch.cuda.synchronize()
    for b, hh in ((0, 0), (77, 41), (143, 95)):
        base = ((b * T + np.arange(T))[:, None] * h + hh * d + np.arange(d)[None]).astype(np.uint64).ravel()
        k = synth.normal_f16(6, synth.STREAM["aux"] + 33, sigma=1.0, index=base).reshape(T, d)
        v = synth.normal_f16(6, synth.STREAM["aux"] + 34, sigma=1.0, index=base).reshape(T, d)
        q = synth.normal_f16(6, synth.STREAM["aux"] + 35, sigma=1.0 / d ** 0.5, index=base).reshape(T, d)
        kh = oracle.dequant_f64(*oracle.quantize(k))[None, None]
        vh = oracle.dequant_f64(*oracle.quantize(v))[None, None]
        ref = oracle.attention_prefill_causal(q.astype(np.float64)[None, None], kh, vh)[0, 0]
        got = host(out[b * T:(b + 1) * T, hh * d:(hh + 1) * d])
        assert_close(got, ref, rel=2e-3, abs_=4e-3, what=f"prefill full-size b={b} h={hh}")
