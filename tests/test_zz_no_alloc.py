"""fq_dequant_gemm_noalloc (split-K partials in the library's fixed per-GPU
scratch, no device allocation) against fq_dequant_gemm on the same inputs:
two calls in a row, the second smaller, bit-identical outputs, no change in
the device's free memory, and a shape whose partials exceed the scratch
rejected with a clear error before any launch."""
import ctypes

import pytest
import torch

from tests._util import log

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")


def _free_bytes():
    hip = ctypes.CDLL("libamdhip64.so")
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _packed(n, k, stream_id):
    w = torch.empty((n, k), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(w, 11, stream_id, 0.02)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device="cuda:0")
    fq.fq_quantize(w, codes, meta)
    return fq.weight_packed(codes, meta, n, k)


def _act(m, k, stream_id, sigma=1.0):
    a = torch.empty((m, k), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(a, 11, stream_id, sigma)
    return a


def test_noalloc_matches_dequant_gemm_twice_then_smaller():
    E = fq
    cases = [  # (M, N, K, epilogue): decode-size products that split K
        (144, 12288, 49152, E.FQ_EPI_BIAS | E.FQ_EPI_RESIDUAL),   # OPT-175B FC2 at batch 144
        (64, 4096, 12288, E.FQ_EPI_BIAS | E.FQ_EPI_RELU),          # smaller, second call
    ]
    prepared = []
    for i, (M, N, K, epi) in enumerate(cases):
        W = _packed(N, K, 100 + i)
        A = _act(M, K, 110 + i)
        bias = _act(1, N, 120 + i, 0.02)[0]
        res = _act(M, N, 130 + i)
        ref = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
        fq.fq_dequant_gemm(A, W, ref, bias=bias, residual=res if epi & E.FQ_EPI_RESIDUAL else None, epilogue=epi)
        prepared.append((M, N, K, epi, W, A, bias, res, ref))
    outs = [torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
            for M, N, K, epi, W, A, bias, res, ref in prepared]
    torch.cuda.synchronize()
    free0 = _free_bytes()
    for (M, N, K, epi, W, A, bias, res, ref), out in zip(prepared, outs):
        log(f"noalloc M={M} N={N} K={K}")
        fq.fq_dequant_gemm_noalloc(A, W, out, bias=bias, residual=res if epi & E.FQ_EPI_RESIDUAL else None,
                                   epilogue=epi)
    torch.cuda.synchronize()
    assert _free_bytes() == free0, "the allocation-free call changed the device's free memory"
    for (M, N, K, epi, W, A, bias, res, ref), out in zip(prepared, outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"M={M} N={N} K={K}"


def test_noalloc_rejects_partials_beyond_the_scratch():
    """M 256, N 36864, K 12288 (the OPT-175B QKV product at batch 256): the
    decode kernel's stream-K schedule needs two fp32 partial slabs, 72 MiB,
    above the 64 MiB scratch: rejected before any launch (the buffers are
    never read)."""
    M, N, K = 256, 36864, 12288
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((N, K // 64, 2), dtype=torch.float16, device="cuda:0")
    W = fq.weight_packed(codes, meta, N, K)
    A = torch.empty((M, K), dtype=torch.float16, device="cuda:0")
    out = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    with pytest.raises(fq.FqError) as e:
        fq.fq_dequant_gemm_noalloc(A, W, out)
    assert e.value.status == fq.FQ_ERR_INVALID and "scratch" in str(e.value)
