"""Dequant-fused GEMM (4-bit and fp16 weights, every epilogue) against the
oracle's float64 GEMM on the reconstructed weights."""
import numpy as np
import pytest
import torch

import synth
from synth.gen import layer_stream
import oracle
from tests._util import dev, host, log

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")


def _tol_check(got, ref64, what):
    """fp16 output of an fp32-accumulated GEMM: within one fp16 rounding plus
    a small accumulation error of the float64 value."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref64)
    bound = np.abs(ref64) * 2.0 ** -11 + 2e-3 * (np.abs(ref64).max() + 1e-3) * 1e-2 + 1e-6
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} beyond bound, max err {err.max():.3e}"


def _run(M, N, K, flags, packed=True, seed=0, qcols=0, f32out=False):
    a = synth.normal_f16(seed, synth.STREAM["aux"] + 1, (M, K), 1.0)
    w = synth.normal_f16(seed, synth.STREAM["aux"] + 2, (N, K), 0.02)
    b = synth.normal_f16(seed, synth.STREAM["aux"] + 3, (N,), 0.1)
    r = synth.normal_f16(seed, synth.STREAM["aux"] + 4, (M, N), 1.0)
    if packed:
        c, m = oracle.quantize(w)
        wref = oracle.dequant_f16(c, m)
        W = fq.weight_packed(dev(c), dev(m), N, K)
        keep = (W,)
    else:
        wref = w
        wd = dev(w)
        W = fq.weight_f16(wd)
        keep = (wd,)
    out = torch.empty((M, N), dtype=torch.float32 if f32out else torch.float16, device="cuda:0")
    ad, bd, rd = dev(a), dev(b), dev(r)
    if f32out:
        flags |= fq.FQ_EPI_F32OUT
    fq.fq_dequant_gemm(ad, W, out, bias=bd, residual=rd, epilogue=flags, qscale=0.125, qscale_cols=qcols)
    torch.cuda.synchronize()
    ref = oracle.gemm(a, wref, b if flags & fq.FQ_EPI_BIAS else None)
    if flags & fq.FQ_EPI_QSCALE:
        ref[:, :qcols] *= 0.125
    if flags & fq.FQ_EPI_RELU:
        ref = np.maximum(ref, 0)
    if flags & fq.FQ_EPI_RESIDUAL:
        ref = ref + r.astype(np.float64)
    del keep
    return host(out), ref


@pytest.mark.parametrize("M", [1, 8, 37, 64, 144, 200, 256, 300])
@pytest.mark.parametrize("N,K", [(64, 256), (200, 1024), (768, 256)])
def test_gemm_packed_shapes(M, N, K):
    log(f"gemm packed M={M} N={N} K={K}")
    got, ref = _run(M, N, K, fq.FQ_EPI_BIAS)
    _tol_check(got, ref, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [64, 90, 100, 144, 256])
@pytest.mark.parametrize("K", [2048, 384])
def test_gemm_decode_kernels(M, K):
    """The 4-bit decode kernels over ragged N and split K: K = 2048 (32 steps,
    a multiple of 4) takes the one-wave-per-SIMD kernel ({min, scale} copied 4
    steps at a time), K = 384 (6 steps) the two-waves-per-SIMD kernel with
    per-step {min, scale} copies."""
    got, ref = _run(M, 1000, K, fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL, seed=M)
    _tol_check(got, ref, f"decode kernel M={M} K={K}")


@pytest.mark.parametrize("M", [200, 256])
def test_gemm_decode_stream_k_ragged(M):
    """The decode kernel's stream-K schedule (one block per CU, each running an
    equal share of (256-column tile, K step) units; a tile's partial slabs
    summed in block order): N = 1003 (a ragged last tile), K = 32768 (512
    steps, 32 segments per tile), two row groups of 128 (the second partly
    past M at 200 rows), bias and residual in the reduction's epilogue."""
    log(f"gemm decode stream-K M={M} N=1003 K=32768")
    got, ref = _run(M, 1003, 32768, fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL, seed=M + 5)
    _tol_check(got, ref, f"stream-K M={M}")


@pytest.mark.parametrize("M,packed", [(5, True), (144, True), (37, False)])
def test_gemm_splitk_ragged_n(M, packed):
    """Split K with N not a multiple of 8: the reduction's scalar path, the
    epilogue's ragged last chunk (bias, residual)."""
    log(f"gemm split-K ragged N M={M} packed={packed}")
    got, ref = _run(M, 1003, 2048, fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL, packed=packed, seed=M + 3)
    _tol_check(got, ref, f"split-K ragged N M={M}")


@pytest.mark.parametrize("M,N,K", [(64, 1000, 2048), (90, 1000, 2048), (100, 1000, 2048), (144, 1000, 2048),
                                   (256, 1000, 2048), (2100, 3900, 512)])
def test_gemm_meta_alignment_fallback(M, N, K):
    """A {min, scale} array that is 4- but not 16-byte aligned takes the kernels
    that copy it 4 bytes per row: at decode sizes the two-waves-per-SIMD
    kernel, which gives lane group g of k slice s the same k chunk (2 g + s)
    and splits K like the one-wave-per-SIMD kernel the aligned array takes, so
    the two outputs agree bit for bit at every row-block count (4, 6, 8, 9,
    two groups of 8); at prefill sizes the 256 x 128 kernel, held to the
    oracle."""
    log(f"gemm meta alignment M={M} N={N} K={K}")
    a = synth.normal_f16(23, synth.STREAM["aux"] + 1, (M, K), 1.0)
    w = synth.normal_f16(23, synth.STREAM["aux"] + 2, (N, K), 0.02)
    c, m = oracle.quantize(w)
    cd, md = dev(c), dev(m)
    ad = dev(a)
    out1 = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(ad, fq.weight_packed(cd, md, N, K), out1)
    flat = torch.zeros(md.numel() + 2, dtype=torch.float16, device="cuda:0")
    flat[2:] = md.reshape(-1)
    m_off = flat[2:].view(md.shape)  # 4 bytes past a 256-byte-aligned allocation
    assert m_off.data_ptr() % 16 == 4
    out2 = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(ad, fq.weight_packed(cd, m_off, N, K), out2)
    torch.cuda.synchronize()
    ref = oracle.gemm(a, oracle.dequant_f16(c, m))
    if M <= 256:
        assert torch.equal(out1, out2)
    _tol_check(host(out1), ref, "meta alignment, aligned")
    _tol_check(host(out2), ref, "meta alignment, 4-byte aligned")


@pytest.mark.parametrize("flags,qcols", [
    (fq.FQ_EPI_BIAS | fq.FQ_EPI_QSCALE, 96),
    (fq.FQ_EPI_BIAS | fq.FQ_EPI_RELU, 0),
    (fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL, 0),
    (0, 0),
])
def test_gemm_epilogues(flags, qcols):
    for M in (16, 260):
        got, ref = _run(M, 192, 512, flags, qcols=qcols)
        _tol_check(got, ref, f"flags={flags} M={M}")


@pytest.mark.parametrize("M", [3, 144, 257])
def test_gemm_fp16_weight_and_f32_out(M):
    got, ref = _run(M, 328, 256, fq.FQ_EPI_BIAS, packed=False, f32out=True)
    err = np.abs(got - ref)
    assert err.max() <= 1e-5 * (np.abs(ref).max() + 1), err.max()
    got, ref = _run(M, 328, 256, fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL, packed=False)
    _tol_check(got, ref, "fp16 weight")


def test_gemm_grid_exact_weight_equals_plain_fp16_gemm():
    """Weights on their own 4-bit grid: the packed GEMM and the fp16-weight GEMM
    must give identical results (same accumulation order, same inputs)."""
    rng = np.random.default_rng(0)
    N, K, M = 128, 512, 70
    codes = rng.integers(0, 16, (N, K))
    codes[:, ::64] = 0
    codes[:, 1::64] = 15
    mn = -rng.integers(1, 16, (N, K // 64)) / 8.0
    s = 2.0 ** -rng.integers(3, 7, (N, K // 64))
    w = (mn.repeat(64, 1) + codes * s.repeat(64, 1)).astype(np.float16)
    c, m = oracle.quantize(w)
    assert np.array_equal(oracle.dequant_f16(c, m), w)
    a = synth.normal_f16(0, 5, (M, K), 1.0)
    outp = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    outf = torch.empty_like(outp)
    ad, wd, cd, md = dev(a), dev(w), dev(c), dev(m)
    fq.fq_dequant_gemm(ad, fq.weight_packed(cd, md, N, K), outp, epilogue=fq.FQ_EPI_F32OUT)
    fq.fq_dequant_gemm(ad, fq.weight_f16(wd), outf, epilogue=fq.FQ_EPI_F32OUT)
    torch.cuda.synchronize()
    assert torch.equal(outp, outf)


@pytest.mark.parametrize("packed", [True, False])
def test_gemm_large_tile_kernel_ragged(packed):
    """M and N not multiples of the large-M tiles, enough tiles to select them
    (4-bit weights: the 256 x 256 kernel; fp16 weights: the 256 x 128 one);
    N = 3900 takes the element-wise epilogue, N = 32776 the 8-wide one with
    a last tile 8 columns wide."""
    log(f"gemm large-tile ragged packed={packed}")
    got, ref = _run(2100, 3900, 256, fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL, packed=packed)
    _tol_check(got, ref, "large tile ragged")
    got, ref = _run(1030, 32776, 128, fq.FQ_EPI_BIAS | fq.FQ_EPI_RELU, packed=packed)
    _tol_check(got, ref, "large tile ragged 2")


def test_gemm_large_tile_vector_epilogue():
    """256 x 256 kernel, 8-wide epilogue with bias + residual, and with the
    query scaling boundary inside an 8-column chunk and fp32 output."""
    log("gemm large-tile vector epilogue")
    got, ref = _run(2100, 4096, 256, fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL)
    _tol_check(got, ref, "vector epilogue")
    got, ref = _run(2100, 4104, 384, fq.FQ_EPI_BIAS | fq.FQ_EPI_QSCALE, qcols=1000, f32out=True)
    _tol_check(got, ref, "vector epilogue qscale f32")


@pytest.mark.parametrize("M,N,K,flags,f32", [
    (2100, 3900, 512, "bias|residual|relu", False),
    (2049, 4104, 256, "bias|qscale", True),
    (4096, 8192, 1024, "bias", False),
])
def test_gemm_256_kernel_epilogues(M, N, K, flags, f32):
    """The 256 x 256 kernel (one wave per SIMD, weight operand rebuilt in
    registers) ragged in M and N, every epilogue, fp16 and fp32 output, within
    the oracle bound; and K = 384 (not a multiple of 256), which the 256 x 128
    kernel takes instead."""
    fl = 0
    for f in flags.split("|"):
        fl |= {"bias": fq.FQ_EPI_BIAS, "residual": fq.FQ_EPI_RESIDUAL, "relu": fq.FQ_EPI_RELU,
               "qscale": fq.FQ_EPI_QSCALE}[f]
    for k in (K, 384):
        log(f"gemm 256 kernel M={M} N={N} K={k} {flags} f32={f32}")
        got, ref = _run(M, N, k, fl, seed=13, qcols=1000, f32out=f32)
        _tol_check(got, ref, f"256 kernel K={k}")


def test_gemm_packed_256x128_kernel():
    """4-bit weights with K not a multiple of 128 take the 256 x 128 kernel."""
    log("gemm packed 256x128 K=192")
    got, ref = _run(2100, 4000, 192, fq.FQ_EPI_BIAS | fq.FQ_EPI_RELU)
    _tol_check(got, ref, "packed 256x128")


@pytest.mark.parametrize("packed", [True, False])
@pytest.mark.parametrize("M", [700, 4100])
def test_gemm_mid_and_large_m_tiles(packed, M):
    """M = 700 (between the decode and the prefill sizes) takes the 128 x 128
    kernel; M = 4100 (ragged) the large-tile kernels (256 x 256 for packed
    weights, 256 x 128 for fp16)."""
    N, K = 4096, 1024
    got, ref = _run(M, N, K, fq.FQ_EPI_BIAS | fq.FQ_EPI_RELU, packed=packed, seed=11)
    _tol_check(got, ref, f"M={M} packed={packed}")


def test_gemm_empty_m_is_noop():
    W = fq.weight_f16(torch.zeros((64, 64), dtype=torch.float16, device="cuda:0"))
    out = torch.full((1, 64), 7.0, dtype=torch.float16, device="cuda:0")
    a = torch.zeros((1, 64), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(a[:0], W, out[:0])
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("M,which", [(144, "w_qkv"), (144, "w_fc1"), (144, "w_fc2"), (8192, "w_fc1")])
def test_gemm_full_size_sampled(M, which):
    """OPT-175B projection shapes (h = 12288, F = 49152) in the launch
    configuration of the decode (M = 144: QKV and FC1 on the decode kernel's
    stream-K schedule, FC2 split K) and prefill-chunk (M = 8192) steps;
    weights generated on the GPU and quantised there; sampled outputs (the
    first and last column of 16 random 256-column tiles among them) against
    float64 dot products of the oracle's reconstruction of the same rows."""
    h, F = 12288, 49152
    N, K = {"w_qkv": (3 * h, h), "w_fc2": (h, F), "w_fc1": (F, h)}[which]
    log(f"gemm full-size M={M} N={N} K={K}")
    sw = layer_stream(3, which)
    w = torch.empty((N, K), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(w, 0, sw, 0.02)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((N, K // 64, 2), dtype=torch.float16, device="cuda:0")
    fq.fq_quantize(w, codes, meta)
    del w
    a = torch.empty((M, K), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(a, 0, synth.STREAM["hidden"], 1.0)
    out = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(a, fq.weight_packed(codes, meta, N, K), out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    tiles = rng.integers(0, N // 256, 16) * 256
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 10), tiles, tiles + 255]))
    ai = (rows[:, None] * K + np.arange(K)[None]).astype(np.uint64).ravel()
    wi = (cols[:, None] * K + np.arange(K)[None]).astype(np.uint64).ravel()
    arows = synth.normal_f16(0, synth.STREAM["hidden"], sigma=1.0, index=ai).reshape(len(rows), K)
    wrows = synth.normal_f16(0, sw, sigma=0.02, index=wi).reshape(len(cols), K)
    ref = oracle.gemm(arows, oracle.dequant_f16(*oracle.quantize(wrows)))
    got = host(out[torch.as_tensor(rows, device="cuda:0")][:, torch.as_tensor(cols, device="cuda:0")])
    _tol_check(got, ref, f"{which} M={M}")


@pytest.mark.parametrize("M,N,K", [(2100, 3900, 512), (2100, 3900, 384), (144, 1024, 512)])
def test_gemm_strided_operands(M, N, K):
    """A, C and the residual with row strides beyond their widths (A padded by
    64 columns, C and the residual by 8): the one-wave-per-SIMD 256 x 256
    kernel, the 256 x 128 one (K = 384) and the decode kernel (M = 144) give
    exactly the contiguous call's output, untouched padding, and stay within
    the oracle bound."""
    log(f"gemm strided M={M} N={N} K={K}")
    a = synth.normal_f16(21, synth.STREAM["aux"] + 1, (M, K), 1.0)
    w = synth.normal_f16(21, synth.STREAM["aux"] + 2, (N, K), 0.02)
    b = synth.normal_f16(21, synth.STREAM["aux"] + 3, (N,), 0.1)
    r = synth.normal_f16(21, synth.STREAM["aux"] + 4, (M, N), 1.0)
    c, m = oracle.quantize(w)
    W = fq.weight_packed(dev(c), dev(m), N, K)
    flags = fq.FQ_EPI_BIAS | fq.FQ_EPI_RESIDUAL
    ad, bd, rd = dev(a), dev(b), dev(r)
    out = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(ad, W, out, bias=bd, residual=rd, epilogue=flags)
    a_pad = torch.zeros((M, K + 64), dtype=torch.float16, device="cuda:0")
    a_pad[:, :K] = ad
    r_pad = torch.zeros((M, N + 8), dtype=torch.float16, device="cuda:0")
    r_pad[:, :N] = rd
    c_pad = torch.full((M, N + 8), 3.0, dtype=torch.float16, device="cuda:0")
    fq.fq_dequant_gemm(a_pad[:, :K], W, c_pad[:, :N], bias=bd, residual=r_pad[:, :N], epilogue=flags)
    torch.cuda.synchronize()
    assert torch.equal(out, c_pad[:, :N]), "strided operands change the result"
    assert (c_pad[:, N:] == 3.0).all(), "padding columns of C written"
    ref = oracle.gemm(a, oracle.dequant_f16(c, m), b) + r.astype(np.float64)
    _tol_check(host(out), ref, "strided")
