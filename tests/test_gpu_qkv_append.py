"""QKV projection with the K/V append fused into the GEMM epilogue
(fq_qkv_gemm_append) against the two-call form (fq_dequant_gemm, then
fq_kv_append) bit for bit, and its cache codes against the oracle's
quantisation of the same fp16 keys and values."""
import numpy as np
import pytest
import torch

import synth
import oracle
from tests._util import dev, host, bits16, log

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")


def _cache(fmt, batch, H, cap, d):
    if fmt == "q4":
        t = (torch.zeros((batch, H, cap, d // 2), dtype=torch.uint8, device="cuda:0"),
             torch.zeros((batch, H, cap, d // 64, 2), dtype=torch.float16, device="cuda:0"))
        t = t + (torch.zeros_like(t[0]), torch.zeros_like(t[1]))
        return fq.kv_layer_view(*t), t
    t = (torch.zeros((batch, H, cap, d), dtype=torch.float16, device="cuda:0"),
         torch.zeros((batch, H, cap, d), dtype=torch.float16, device="cuda:0"))
    return fq.kv_layer_view_f16(*t), t


# (H, d, B, T, pos, b0, fmt): the first three take a fused 256 x 256 kernel
# (ragged M = 2100 in the second), the last one the two-call fallback (small M).
CASES = [(8, 128, 4, 1024, 0, 0, "q4"), (12, 128, 3, 700, 5, 1, "q4"), (16, 64, 4, 1024, 3, 0, "f16"),
         (4, 64, 2, 5, 2, 1, "q4")]


@pytest.mark.parametrize("H,d,B,T,pos,b0,fmt", CASES)
def test_fused_append_equals_two_calls(H, d, B, T, pos, b0, fmt):
    _fused_vs_two_calls(H, d, B, T, pos, b0, fmt)



def _fused_vs_two_calls(H, d, B, T, pos, b0, fmt):
    h = H * d
    M, K, N = B * T, h, 3 * h
    log(f"qkv append H={H} d={d} B={B} T={T} pos={pos} b0={b0} {fmt} (M={M})")
    a = synth.normal_f16(7, synth.STREAM["aux"] + 40, (M, K), 1.0)
    w = synth.normal_f16(7, synth.STREAM["aux"] + 41, (N, K), 0.02)
    bias = synth.normal_f16(7, synth.STREAM["aux"] + 42, (N,), 0.1)
    c, m = oracle.quantize(w)
    W = fq.weight_packed(dev(c), dev(m), N, K)
    ad, bd = dev(a), dev(bias)
    qscale = d ** -0.5
    batch, cap = b0 + B + 1, pos + T + 3
    # two-call form
    view1, keep1 = _cache(fmt, batch, H, cap, d)
    c1 = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(ad, W, c1, bias=bd, epilogue=fq.FQ_EPI_BIAS | fq.FQ_EPI_QSCALE, qscale=qscale, qscale_cols=h)
    fq.fq_kv_append(view1, c1[:, h:], c1[:, 2 * h:], N, b0, B, T, pos)
    # fused form
    view2, keep2 = _cache(fmt, batch, H, cap, d)
    c2 = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda:0")
    fq.fq_qkv_gemm_append(ad, W, bd, qscale, view2, b0, B, T, pos, c2)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(host(c1[:, :h])), bits16(host(c2[:, :h]))), "q columns differ"
    for t1, t2 in zip(keep1, keep2):
        x1, x2 = host(t1), host(t2)
        if x1.dtype == np.float16:
            x1, x2 = bits16(x1), bits16(x2)
        assert np.array_equal(x1, x2), "cache contents differ"
    # the oracle's quantisation of the fp16 K and V the projection produced
    if fmt == "q4":
        kc, km, vc, vm = (host(t) for t in keep2)
        for cols, codes, meta in ((slice(h, 2 * h), kc, km), (slice(2 * h, 3 * h), vc, vm)):
            x = host(c1[:, cols]).reshape(B, T, H, d).transpose(0, 2, 1, 3)
            rc, rm = oracle.quantize(np.ascontiguousarray(x))
            assert np.array_equal(codes[b0:b0 + B, :, pos:pos + T], rc)
            assert np.array_equal(bits16(meta[b0:b0 + B, :, pos:pos + T]), bits16(rm))
        assert not kc[:b0].any() and not kc[b0:b0 + B, :, :pos].any() and not vm[b0:b0 + B, :, pos + T:].any()
    else:
        k16, v16 = (host(t) for t in keep2)
        x = host(c1[:, h:2 * h]).reshape(B, T, H, d).transpose(0, 2, 1, 3)
        assert np.array_equal(bits16(k16[b0:b0 + B, :, pos:pos + T]), bits16(x))
        assert not k16[b0:b0 + B, :, :pos].any() and not v16[b0 + B:].any()


def test_fused_append_argument_errors():
    H, d = 2, 64
    h = H * d
    view, keep = _cache("q4", 2, H, 8, d)
    W = fq.weight_packed(torch.zeros((3 * h, h // 2), dtype=torch.uint8, device="cuda:0"),
                         torch.zeros((3 * h, h // 64, 2), dtype=torch.float16, device="cuda:0"), 3 * h, h)
    a = torch.zeros((4, h), dtype=torch.float16, device="cuda:0")
    c = torch.zeros((4, 3 * h), dtype=torch.float16, device="cuda:0")
    with pytest.raises(fq.FqError):   # M != B * T
        fq.fq_qkv_gemm_append(a, W, None, 1.0, view, 0, 2, 3, 0, c)
    with pytest.raises(fq.FqError):   # positions beyond the capacity
        fq.fq_qkv_gemm_append(a, W, None, 1.0, view, 0, 2, 2, 7, c)
    W2 = fq.weight_packed(torch.zeros((2 * h, h // 2), dtype=torch.uint8, device="cuda:0"),
                          torch.zeros((2 * h, h // 64, 2), dtype=torch.float16, device="cuda:0"), 2 * h, h)
    with pytest.raises(fq.FqError):   # W is not [3h, K]
        fq.fq_qkv_gemm_append(a, W2, None, 1.0, view, 0, 2, 2, 0, c)


def test_fused_append_full_size():
    """OPT-175B QKV projection in the prompt pass's launch configuration: a
    16384-row chunk (32 sequences x 512 tokens, sequences 32..63 of a 64-sequence
    cache), h = 12288, weights generated and quantised on the GPU.  The fused
    form equals the two-call form on every q value and cache byte; sampled
    groups match the oracle's quantisation of the projection's fp16 K/V."""
    from synth.gen import layer_stream
    H, d, B, T, b0 = 96, 128, 32, 512, 32
    h = H * d
    M, N, K = B * T, 3 * h, h
    log("qkv append full-size")
    w = torch.empty((N, K), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(w, 0, layer_stream(0, "w_qkv"), 0.02)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((N, K // 64, 2), dtype=torch.float16, device="cuda:0")
    fq.fq_quantize(w, codes, meta)
    del w
    W = fq.weight_packed(codes, meta, N, K)
    a = torch.empty((M, K), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(a, 0, synth.STREAM["hidden"], 1.0)
    bias = torch.empty((N,), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(bias, 0, layer_stream(0, "b_qkv"), 0.02)
    view1, keep1 = _cache("q4", 64, H, T, d)
    c1 = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(a, W, c1, bias=bias, epilogue=fq.FQ_EPI_BIAS | fq.FQ_EPI_QSCALE, qscale=d ** -0.5,
                       qscale_cols=h)
    fq.fq_kv_append(view1, c1[:, h:], c1[:, 2 * h:], N, b0, B, T, 0)
    view2, keep2 = _cache("q4", 64, H, T, d)
    c2 = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_qkv_gemm_append(a, W, bias, d ** -0.5, view2, b0, B, T, 0, c2)
    torch.cuda.synchronize()
    assert torch.equal(c1[:, :h], c2[:, :h]), "q columns differ"
    for t1, t2 in zip(keep1, keep2):
        assert torch.equal(t1, t2), "cache contents differ"
    kc, km = keep2[0], keep2[1]
    for b, t, hh in ((0, 0, 0), (17, 300, 50), (31, 511, 95)):
        x = host(c1[b * T + t, h + hh * d:h + (hh + 1) * d]).reshape(1, d)
        rc, rm = oracle.quantize(x)
        assert np.array_equal(host(kc[b0 + b, hh, t]), rc[0])
        assert np.array_equal(bits16(host(km[b0 + b, hh, t])), bits16(rm[0]))


def test_fused_append_empty_and_head_dim_64_fused_path():
    """M = 0 (no sequences or no tokens) is a no-op that leaves the cache and C
    untouched; head_dim 64 through the fused kernel (4 heads share a 256-wide
    tile) equals the two-call form."""
    H, d = 16, 64
    h = H * d
    view, keep = _cache("q4", 2, H, 8, d)
    W = fq.weight_packed(torch.zeros((3 * h, h // 2), dtype=torch.uint8, device="cuda:0"),
                         torch.zeros((3 * h, h // 64, 2), dtype=torch.float16, device="cuda:0"), 3 * h, h)
    a = torch.zeros((0, h), dtype=torch.float16, device="cuda:0")
    c = torch.full((1, 3 * h), 5.0, dtype=torch.float16, device="cuda:0")
    fq.fq_qkv_gemm_append(a, W, None, 1.0, view, 0, 0, 4, 0, c)   # B = 0
    fq.fq_qkv_gemm_append(a, W, None, 1.0, view, 0, 2, 0, 0, c)   # T = 0
    torch.cuda.synchronize()
    assert (c == 5.0).all() and not any(t.any() for t in keep)
    _fused_vs_two_calls(16, 64, 2, 2048, 4, 1, "q4")


def test_decode_attention_length_limit_and_empty_batch():
    """Lengths beyond the score buffer are refused on the host; B = 0 is a no-op."""
    H, d = 2, 64
    view, keep = _cache("q4", 1, H, 30001, d)
    q = torch.zeros((1, H * d), dtype=torch.float16, device="cuda:0")
    out = torch.full((1, H * d), 3.0, dtype=torch.float16, device="cuda:0")
    with pytest.raises(fq.FqError):
        fq.fq_decode_attention(q, view, 0, 1, 30001, out)
    fq.fq_decode_attention(q, view, 0, 0, 5, out)
    torch.cuda.synchronize()
    assert (out == 3.0).all()
