"""GPU quantiser, reconstruction, quantise-on-append and the shared input
generator against the CPU oracle: bit-exact codes and fp16 {min, scale}."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from synth.gen import layer_stream
import oracle
from tests._util import dev, host, empty_packed, bits16, log

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")


def _gpu_quant(x16_dev):
    rows, cols = x16_dev.shape
    codes, meta = empty_packed(rows, cols)
    fq.fq_quantize(x16_dev, codes, meta)
    torch.cuda.synchronize()
    return host(codes), host(meta)


def test_synth_generator_matches_numpy():
    # 4M elements per sigma: a double- versus single-rounding difference in the
    # fp32 product -> fp16 step shows up about once per 30k elements
    for sigma, n, first in ((0.02, 4_000_003, 0), (1.0, 4_000_000, 12345)):
        d = torch.empty(n, dtype=torch.float16, device="cuda:0")
        fq.fq_synth_normal_f16(d, 7, 99, sigma, first=first)
        ref = synth.normal_f16(7, 99, sigma=sigma, index=np.arange(first, first + n, dtype=np.uint64))
        assert np.array_equal(bits16(host(d)), bits16(ref))
    ids = torch.empty(5000, dtype=torch.int32, device="cuda:0")
    fq.fq_synth_token_ids(ids, 3, synth.STREAM["prompt"], 50272)
    assert np.array_equal(host(ids), synth.token_ids(3, synth.STREAM["prompt"], (5000,), 50272))


@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 256), (300, 4096), (129, 1024)])
def test_quantize_bit_exact(rows, cols):
    log(f"quantize rows={rows} cols={cols}")
    x = synth.normal_f16(0, synth.STREAM["aux"] + rows, (rows, cols), 0.02)
    c, m = _gpu_quant(dev(x))
    rc, rm = oracle.quantize(x)
    assert np.array_equal(c, rc)
    assert np.array_equal(bits16(m), bits16(rm))


def test_quantize_worked_examples_and_degenerate_groups():
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_worked_examples.json")))
    rows = []
    for g in gold["groups"]:
        if g.get("x") == "ramp16":
            x = np.arange(64) % 16
        else:
            x = np.full(64, g["fill"])
            x[:len(g["x_head"])] = g["x_head"]
        rows.append(x.astype(np.float16))
    # extra: negative zero mixes, huge range, tiny values, all-negative
    rows.append(np.where(np.arange(64) % 3 == 0, -0.0, 0.0).astype(np.float16))
    rows.append(np.linspace(-65504, 65504, 64).astype(np.float16))
    rows.append((np.arange(64) * 6e-8).astype(np.float16))
    rows.append(-np.abs(synth.normal_f16(1, 5, (64,), 1.0)))
    x = np.stack(rows)
    c, m = _gpu_quant(dev(x))
    rc, rm = oracle.quantize(x)
    assert np.array_equal(c, rc)
    assert np.array_equal(bits16(m), bits16(rm))
    for i, g in enumerate(gold["groups"]):
        assert int(bits16(m)[i, 0, 0]) == int(g["min_bits"], 16)
        assert int(bits16(m)[i, 0, 1]) == int(g["scale_bits"], 16)


def test_quantize_strided_and_unaligned_rows():
    base = synth.normal_f16(0, 77, (20, 200), 1.0)
    xd = dev(base)[:, 4:4 + 128]          # row stride 200 (not a multiple of 8), offset 4 elements
    c, m = _gpu_quant(xd)
    rc, rm = oracle.quantize(np.ascontiguousarray(base[:, 4:132]))
    assert np.array_equal(c, rc) and np.array_equal(bits16(m), bits16(rm))


def test_dequantize_bit_exact():
    x = synth.normal_f16(0, 78, (65, 512), 0.02)
    c, m = oracle.quantize(x)
    y = torch.empty((65, 512), dtype=torch.float16, device="cuda:0")
    fq.fq_dequantize(dev(c), dev(m), 65, 512, y)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(host(y)), bits16(oracle.dequant_f16(c, m)))


@pytest.mark.parametrize("H,d,B,T,pos", [(4, 64, 3, 5, 0), (4, 128, 2, 1, 9), (32, 128, 2, 7, 3)])
def test_kv_append_bit_exact(H, d, B, T, pos):
    h = H * d
    cap = pos + T + 2
    qkv = synth.normal_f16(2, 90 + H, (B * T, 3 * h), 1.0)
    qd = dev(qkv)
    kc = torch.zeros((B + 1, H, cap, d // 2), dtype=torch.uint8, device="cuda:0")
    km = torch.zeros((B + 1, H, cap, d // 64, 2), dtype=torch.float16, device="cuda:0")
    vc, vm = torch.zeros_like(kc), torch.zeros_like(km)
    view = fq.kv_layer_view(kc, km, vc, vm)
    fq.fq_kv_append(view, qd[:, h:], qd[:, 2 * h:], 3 * h, 1, B, T, pos)
    torch.cuda.synchronize()
    k = qkv[:, h:2 * h].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    v = qkv[:, 2 * h:].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    rkc, rkm = oracle.quantize(np.ascontiguousarray(k))
    rvc, rvm = oracle.quantize(np.ascontiguousarray(v))
    assert np.array_equal(host(kc)[1:, :, pos:pos + T], rkc)
    assert np.array_equal(bits16(host(km)[1:, :, pos:pos + T]), bits16(rkm))
    assert np.array_equal(host(vc)[1:, :, pos:pos + T], rvc)
    assert np.array_equal(bits16(host(vm)[1:, :, pos:pos + T]), bits16(rvm))
    # untouched entries stay zero
    assert not host(kc)[0].any() and not host(kc)[1:, :, :pos].any()


@pytest.mark.parametrize("H,d,B,T,pos,shift", [(4, 64, 3, 5, 0, 0), (4, 128, 2, 1, 9, 0), (3, 128, 2, 7, 3, 1)])
def test_kv_append_f16_copies_exactly(H, d, B, T, pos, shift):
    """fp16 cache: the new K/V land unchanged at positions pos..pos+T-1 (shift 1
    offsets the source by one element, taking the unaligned path)."""
    h = H * d
    cap = pos + T + 2
    qkv = synth.normal_f16(3, 95 + H, (B * T, 3 * h + shift), 1.0)
    qd = dev(qkv)
    k16 = torch.zeros((B + 1, H, cap, d), dtype=torch.float16, device="cuda:0")
    v16 = torch.zeros_like(k16)
    view = fq.kv_layer_view_f16(k16, v16)
    fq.fq_kv_append(view, qd[:, shift + h:], qd[:, shift + 2 * h:], 3 * h + shift, 1, B, T, pos)
    torch.cuda.synchronize()
    k = qkv[:, shift + h:shift + 2 * h].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    v = qkv[:, shift + 2 * h:].reshape(B, T, H, d).transpose(0, 2, 1, 3)
    assert np.array_equal(bits16(host(k16)[1:, :, pos:pos + T]), bits16(k))
    assert np.array_equal(bits16(host(v16)[1:, :, pos:pos + T]), bits16(v))
    assert not host(k16)[0].any() and not host(k16)[1:, :, :pos].any() and not host(v16)[1:, :, pos + T:].any()


def test_kv_view_format_errors():
    k16 = torch.zeros((1, 2, 4, 64), dtype=torch.float16, device="cuda:0")
    bad = fq.kv_layer_view_f16(k16, torch.zeros_like(k16))
    bad.bits = 7
    x = torch.zeros((1, 3 * 128), dtype=torch.float16, device="cuda:0")
    with pytest.raises(fq.FqError):
        fq.fq_kv_append(bad, x[:, 128:], x[:, 256:], 384, 0, 1, 1, 0)
    with pytest.raises(fq.FqError):
        fq.fq_decode_attention(x, bad, 0, 1, 1, torch.zeros((1, 128), dtype=torch.float16, device="cuda:0"))
    missing = fq.kv_layer_view_f16(k16, torch.zeros_like(k16))
    missing.v16 = None
    with pytest.raises(fq.FqError):
        fq.fq_prefill_attention(x, missing, 0, 1, 1, 0, torch.zeros((1, 128), dtype=torch.float16, device="cuda:0"))


def test_quantize_full_size_weight_sampled_rows():
    """FC1 weight of the OPT-175B shape (49152 x 12288), generated on the GPU;
    sampled rows checked bit-exactly against the oracle on the same inputs."""
    n, k = 49152, 12288
    log(f"quantize full-size {n}x{k}")
    w = torch.empty((n, k), dtype=torch.float16, device="cuda:0")
    fq.fq_synth_normal_f16(w, 0, layer_stream(0, "w_fc1"), 0.02)
    codes, meta = empty_packed(n, k)
    fq.fq_quantize(w, codes, meta)
    torch.cuda.synchronize()
    del w
    rows = np.array([0, 1, 4095, 20000, 49151])
    idx = (rows[:, None] * k + np.arange(k)[None]).astype(np.uint64)
    x = synth.normal_f16(0, layer_stream(0, "w_fc1"), sigma=0.02, index=idx.ravel()).reshape(len(rows), k)
    rc, rm = oracle.quantize(x)
    sel = torch.as_tensor(rows, device="cuda:0")
    assert np.array_equal(host(codes[sel]), rc)
    assert np.array_equal(bits16(host(meta[sel])), bits16(rm))
