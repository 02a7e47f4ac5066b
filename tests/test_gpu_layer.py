"""fq_layer_step (prefill + decode of one OPT-style layer) against the oracle
under teacher forcing (the oracle quantises the GPU's own fp16 K/V, so both
caches hold the same codes): the tiny configuration in full, the
OPT-6.7B-shaped layer on 8 of its 64 sequences at every position, and the
packed weights bit-exact."""
import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import LayerConfig
from tests._util import (dev, host, bits16, assert_close, assert_layer_close, log, gpu_cache, packed_to_host,
                         assert_same_cache)

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")

NAMES = ("w_qkv", "w_out", "w_fc1", "w_fc2", "b_qkv", "b_out", "b_fc1", "b_fc2",
         "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def _check_packed(model, layer, params, cfg):
    for i, name in enumerate(("w_qkv", "w_out", "w_fc1", "w_fc2")):
        codes, meta = packed_to_host(model.packed_weight(layer, i))
        rc, rm = oracle.quantize(params[name], cfg.group)
        gm = bits16(meta)
        bad = np.argwhere(gm != bits16(rm))
        assert len(bad) == 0, f"{name}: {len(bad)} meta mismatches, first {bad[:4].tolist()} " \
                              f"gpu {[gm[tuple(i)] for i in bad[:4]]} oracle {[bits16(rm)[tuple(i)] for i in bad[:4]]}"
        assert np.array_equal(codes, rc), name


def _run_layer(model, kv, hd, B, P, T, cs):
    """Prefill of P tokens in chunks of cs sequences, then T decode steps; returns
    the layer outputs [B, P + T, h] on the host."""
    h = hd.shape[-1]
    x = hd[:, :P].reshape(B * P, h).contiguous()
    y = torch.empty_like(x)
    for b0 in range(0, B, cs):
        nb = min(cs, B - b0)
        fq.fq_layer_step(model, 0, kv, b0, nb, P, 0, x[b0 * P:(b0 + nb) * P], y[b0 * P:(b0 + nb) * P])
    ys = [host(y).reshape(B, P, h)]
    for t in range(T):
        xt = hd[:, P + t].contiguous()
        yt = torch.empty_like(xt)
        fq.fq_layer_step(model, 0, kv, 0, B, 1, P + t, xt, yt)
        ys.append(host(yt).reshape(B, 1, h))
    torch.cuda.synchronize()
    return np.concatenate(ys, 1)


def _layer_case(cfg, B, P, T, seed, bias_sigma, check=None, chunk=None, via_init=False, cache_resident=-1,
                heavy=None):
    """The layer over a prefill of P tokens (in chunks of `chunk` sequences) and T
    decode steps on the GPU, against the oracle under teacher forcing for the
    sequences check = (b0, nb) (default: all):
      - the GPU records the fp16 K/V it appends (fq_model_set_capture); the
        oracle's quantisation of those values equals the GPU cache bit for bit;
      - the GPU's fp16 K/V are within the layer tolerance of the oracle's own
        float64 K/V (a storage point of the layer);
      - every layer output (the prefill block and each decode step) is within
        relative L2 5e-3 and max |err| 3e-2 of the oracle's float64 value while
        it and the residual x1 stay below 16 in magnitude (above that the bound
        grows with their fp16 rounding: assert_layer_close), the oracle
        attending over that same cache (layer_rows);
      - a second GPU run without the capture (so with the K/V append fused into
        the QKV projection at prefill sizes) gives bit-identical outputs and cache.
    heavy: replace the four weight matrices by heavy-tailed draws of that kind
    (synth.heavy_tailed_f16, scale 0.02) -- quantisation groups of wide range."""
    h, H, d = cfg.hidden, cfg.heads, cfg.head_dim
    model = fq.Model(h, cfg.heads, cfg.ffn, 1, max_tokens=max(B * P if chunk is None else chunk * P, B),
                     compress_weight=cfg.compress_weight, compress_cache=cfg.compress_cache,
                     cache_resident_layers=cache_resident)
    params = oracle.layer_params(seed, cfg, 0, bias_sigma, workers=16)
    if heavy is not None:
        for n in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
            params[n] = synth.heavy_tailed_f16(seed, synth.gen.layer_stream(0, n), params[n].shape, 0.02, heavy)
    if via_init:
        model.init_random(seed, bias_sigma)
    else:
        model.set_layer(0, {n: dev(params[n]) for n in NAMES})
    torch.cuda.synchronize()
    if cfg.compress_weight:
        _check_packed(model, 0, params, cfg)
    S = P + T
    b0, nb = check if check is not None else (0, B)
    hidden = synth.normal_f16(seed, synth.STREAM["hidden"], (B, S, h), 1.0)
    hd = dev(hidden)
    cs = B if chunk is None else chunk
    runs = []
    for capture in (True, False):
        kv = fq.KVCache(model, B, S)
        cap = {n: torch.zeros((nb, S, h), dtype=torch.float16, device="cuda:0") for n in ("k16", "v16")}
        model.set_capture([dict(layer=0, b0=b0, nb=nb, capacity=S, **cap)] if capture else [])
        y = _run_layer(model, kv, hd, B, P, T, cs)
        model.set_capture([])
        runs.append((y, gpu_cache(kv.view(0), B, S), {n: host(t) for n, t in cap.items()}))
        kv.close()
    (y, gcache, kvg), (y2, gcache2, _) = runs
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "capture changed the layer's outputs"
    for name in gcache:
        assert np.array_equal(gcache[name].view(np.uint8), gcache2[name].view(np.uint8)), name
    model.close()
    # the oracle's cache holds its quantisation of the GPU's fp16 K/V
    cache = oracle.new_cache(cfg, nb, S)
    oracle.cache_fill(cache, cfg, kvg["k16"], kvg["v16"], 0)
    assert_same_cache({n: g[b0:b0 + nb] for n, g in gcache.items()}, cache, "cache")
    packed = oracle.pack_layer(params, cfg, workers=16)
    r = oracle.layer_rows(hidden[b0:b0 + nb], np.arange(S), params, packed, cache, cfg,
                          want=("k64", "v64", "x1_64"))
    assert_close(kvg["k16"], r["k64"], what="K (fp16 storage point)")
    assert_close(kvg["v16"], r["v64"], what="V (fp16 storage point)")
    yb = y[b0:b0 + nb]
    x1 = np.abs(r["x1_64"])
    rel, mx, mag, _ = assert_layer_close(yb[:, :P], r["y64"][:, :P], x1[:, :P], what="prefill outputs")
    log(f"prefill: rel_l2 {rel:.2e} max_abs {mx:.2e} max |y| {mag:.3g}")
    for t in range(T):
        assert_layer_close(yb[:, P + t], r["y64"][:, P + t], x1[:, P + t], what=f"decode step {t}")


@pytest.mark.parametrize("bias_sigma", [0.0, 0.02])
def test_layer_tiny_config_full(bias_sigma):
    """hidden 256, 4 heads x 64, FFN 1024, batch 8, prompt 64, 4 decode steps, seed 0."""
    log(f"layer tiny bias_sigma={bias_sigma}")
    _layer_case(LayerConfig(256, 4, 1024), B=8, P=64, T=4, seed=0, bias_sigma=bias_sigma)


def test_layer_tiny_via_device_init():
    """Same layer with weights generated and quantised on the GPU."""
    _layer_case(LayerConfig(256, 4, 1024), B=8, P=64, T=4, seed=0, bias_sigma=0.0, via_init=True)


@pytest.mark.parametrize("weight,cache", [(True, False), (False, False), (False, True)])
def test_layer_compression_toggles(weight, cache):
    """Weight-only, neither, and cache-only compression on the tiny layer."""
    log(f"layer tiny compress_weight={weight} compress_cache={cache}")
    cfg = LayerConfig(256, 4, 1024, compress_weight=weight, compress_cache=cache)
    _layer_case(cfg, B=8, P=64, T=4, seed=1, bias_sigma=0.02)


@pytest.mark.parametrize("cache", [True, False])
def test_layer_offloaded_cache(cache):
    """The layer's cache in pinned host memory (staged per call), prefill in
    chunks of 3 sequences then decode steps, 4-bit and fp16 cache."""
    log(f"layer offloaded cache compress_cache={cache}")
    cfg = LayerConfig(256, 4, 1024, compress_cache=cache)
    _layer_case(cfg, B=8, P=64, T=4, seed=2, bias_sigma=0.02, chunk=3, cache_resident=0)


def test_layer_weight_only_ragged_shapes():
    """head_dim 128 with the fp16 cache, ragged prompt and chunked prefill."""
    cfg = LayerConfig(512, 4, 1536, compress_weight=True, compress_cache=False)
    _layer_case(cfg, B=5, P=70, T=3, seed=4, bias_sigma=0.02, chunk=2)


def test_layer_ragged_shapes():
    """head_dim 128, prompt not a multiple of the 64-query tile, odd batch, prefill in
    chunks of 2 sequences; sequences 1-3 (across chunks) checked."""
    log("layer ragged")
    _layer_case(LayerConfig(512, 4, 1536), B=5, P=70, T=3, seed=3, bias_sigma=0.02, chunk=2, check=(1, 3))


@pytest.mark.slow
def test_layer_opt67b_shape_sampled():
    """One OPT-6.7B-shaped layer (hidden 4096, 32 x 128, FFN 16384), batch 64,
    prompt 512 (prefill in chunks of 16 sequences), 32 decode steps; every
    sequence runs on the GPU, sequences 40-47 are checked against the oracle at
    every position."""
    log("layer OPT-6.7B shape")
    _layer_case(LayerConfig(4096, 32, 16384), B=64, P=512, T=32, seed=0, bias_sigma=0.0,
                check=(40, 8), chunk=16, via_init=True)
