"""OPT-style pre-LayerNorm decoder layer and greedy generation over 4-bit weights
and a 4-bit KV cache, evaluated on the CPU.

Pages: FlexGen README (giters.com mirror) -- "Extreme Compression" (4-bit
weights and attention cache), "Benchmark Results" (OPT-6.7B/30B/175B at
prompt 512, output 32; throughput = generated tokens / (prompt time +
generation time)); pith.science abstract (OPT-175B at effective batch 144).
The layer internals (pre-LayerNorm, ReLU FFN, learned positions with the
OPT offset of 2, LM head tied to the token embedding) are the OPT
architecture the pages name; the pages themselves do not spell them out.

fp16 storage points (every value below marked [16] is rounded once to fp16,
round-to-nearest-even, from its float64 value; everything between them is
float64):
  h1 = LN1(x)[16]
  q  = ((h1 Wq^T + bq) * d^-1/2)[16];  k = (h1 Wk^T + bk)[16];  v = (h1 Wv^T + bv)[16]
  k, v appended to the cache as 4-bit groups (quant.quantize), or kept as
  fp16 when cache compression is off, then
  o  = attention(q, dequant(K cache), dequant(V cache))[16]  (the fp16 cache
       is read as stored)
  x1 = (x + o Wo^T + bo)[16]
  h2 = LN2(x1)[16]
  f  = relu(h2 W1^T + b1)[16]
  y  = (x1 + f W2^T + b2)[16]
W^ is dequant_f16 of the packed weight (or the fp16 weight itself when
weights are not compressed).  The new token's K/V enter the cache before
attention, so the query always attends over the reconstructed cache.
Weight and cache compression are separate switches (README, "Handle
Out-of-memory": --compress-weight; Manning "FlexGen technique" page,
"Configuring an OPT model": the policy enables weight and cache compression
separately).
"""
from dataclasses import dataclass

import numpy as np

import synth
from synth.gen import layer_stream

from .quant import quantize, dequant_f16, dequant_f64, GROUP
from .ops import gemm, layernorm, softmax


@dataclass(frozen=True)
class LayerConfig:
    hidden: int
    heads: int
    ffn: int
    group: int = GROUP
    compress_weight: bool = True
    compress_cache: bool = True

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads


@dataclass(frozen=True)
class ModelConfig:
    layer: LayerConfig
    layers: int
    vocab: int
    max_pos: int          # rows of the position table (positions used: pos + 2)


def layer_params(seed: int, cfg: LayerConfig, layer: int, bias_sigma: float = 0.0, workers: int = 1) -> dict:
    """fp16 parameters of one layer from the seeded generator.

    Weights ~ (bounded) N(0, 0.02).  bias_sigma == 0: OPT-style init (biases 0,
    LN gamma 1, beta 0).  bias_sigma > 0: biases and betas ~ N(0, bias_sigma),
    gammas ~ N(0, 1), to exercise every term of the layer.  `workers` threads
    generate the large tensors (same values)."""
    h, F = cfg.hidden, cfg.ffn
    w = lambda name, shape: synth.normal_f16(seed, layer_stream(layer, name), shape, 0.02, workers=workers)
    p = {"w_qkv": w("w_qkv", (3 * h, h)), "w_out": w("w_out", (h, h)),
         "w_fc1": w("w_fc1", (F, h)), "w_fc2": w("w_fc2", (h, F))}
    shapes = {"b_qkv": 3 * h, "b_out": h, "b_fc1": F, "b_fc2": h,
              "ln1_g": h, "ln1_b": h, "ln2_g": h, "ln2_b": h}
    for name, n in shapes.items():
        if bias_sigma > 0:
            sig = 1.0 if name.endswith("_g") else bias_sigma
            p[name] = synth.normal_f16(seed, layer_stream(layer, name), (n,), sig)
        else:
            p[name] = (np.ones if name.endswith("_g") else np.zeros)(n, dtype=np.float16)
    return p


def pack_layer(params: dict, cfg: LayerConfig, workers: int = 1) -> dict:
    """Linear weights as used by the GEMMs: dequant_f16(quantize(W)) when weights are
    compressed, else W itself -- held as float64 (exact copies of the fp16 values)
    so that every GEMM reads them without a conversion.  Also returns the packed
    codes/meta.  Quantisation groups lie within one row, so with `workers` > 1
    blocks of rows are packed on that many threads (same values)."""
    out = {}
    for name in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
        w = params[name]
        if cfg.compress_weight:
            n, k = w.shape
            codes = np.empty((n, k // 2), np.uint8)
            meta = np.empty((n, k // cfg.group, 2), np.float16)
            wd = np.empty((n, k), np.float64)
            rows = max(1, n // (4 * workers)) if workers > 1 else n

            def part(r0, w=w, codes=codes, meta=meta, wd=wd, rows=rows):
                c, m = quantize(w[r0:r0 + rows], cfg.group)
                codes[r0:r0 + rows], meta[r0:r0 + rows] = c, m
                wd[r0:r0 + rows] = dequant_f16(c, m, cfg.group)
            if workers > 1:
                from concurrent.futures import ThreadPoolExecutor
                with ThreadPoolExecutor(workers) as ex:
                    list(ex.map(part, range(0, n, rows)))
            else:
                part(0)
            out[name] = wd
            out[name + ".codes"], out[name + ".meta"] = codes, meta
        else:
            out[name] = w.astype(np.float64)
    return out


def new_cache(cfg: LayerConfig, batch: int, capacity: int) -> dict:
    """Empty 4-bit K/V cache of one layer: codes [B, H, S_cap, d/2], meta [B, H, S_cap, d/g, 2]."""
    H, d, g = cfg.heads, cfg.head_dim, cfg.group
    if cfg.compress_cache:
        return {"k_codes": np.zeros((batch, H, capacity, d // 2), np.uint8),
                "k_meta": np.zeros((batch, H, capacity, d // g, 2), np.float16),
                "v_codes": np.zeros((batch, H, capacity, d // 2), np.uint8),
                "v_meta": np.zeros((batch, H, capacity, d // g, 2), np.float16)}
    return {"k": np.zeros((batch, H, capacity, d), np.float16),
            "v": np.zeros((batch, H, capacity, d), np.float16)}


def _cache_append(cache: dict, cfg: LayerConfig, k16, v16, pos: int) -> None:
    """k16, v16 [B, H, T, d] fp16 -> cache positions pos..pos+T-1 (groups of 64 along d)."""
    T = k16.shape[2]
    if cfg.compress_cache:
        kc, km = quantize(k16, cfg.group)
        vc, vm = quantize(v16, cfg.group)
        cache["k_codes"][:, :, pos:pos + T] = kc
        cache["k_meta"][:, :, pos:pos + T] = km
        cache["v_codes"][:, :, pos:pos + T] = vc
        cache["v_meta"][:, :, pos:pos + T] = vm
    else:
        cache["k"][:, :, pos:pos + T] = k16
        cache["v"][:, :, pos:pos + T] = v16


def _cache_read(cache: dict, cfg: LayerConfig, length: int, b=slice(None)):
    if cfg.compress_cache:
        k = dequant_f64(cache["k_codes"][b, :, :length], cache["k_meta"][b, :, :length], cfg.group)
        v = dequant_f64(cache["v_codes"][b, :, :length], cache["v_meta"][b, :, :length], cfg.group)
        return k, v
    return (cache["k"][b, :, :length].astype(np.float64), cache["v"][b, :, :length].astype(np.float64))


def _attend(q16, cache, cfg: LayerConfig, pos: int):
    """q16 [B, H, T, d]; query t sits at absolute position pos+t and sees keys 0..pos+t."""
    B, H, T, d = q16.shape
    n = pos + T
    out = np.empty((B, H, T, d), np.float64)
    key_pos = np.arange(n)[None, :]
    qry_pos = (pos + np.arange(T))[:, None]
    mask = key_pos > qry_pos                                  # [T, n]
    for b in range(B):
        k, v = _cache_read(cache, cfg, n, b)                  # [H, n, d]
        s = q16[b].astype(np.float64) @ np.swapaxes(k, -1, -2)  # [H, T, n]
        s[:, mask] = -np.inf
        out[b] = softmax(s, axis=-1) @ v
    return out


def _qkv(xf, params, packed, cfg):
    """LN1 and the QKV projection of rows xf [M, h]: h1, q (scaled), k, v at their
    storage points, plus k and v in float64 before rounding."""
    h, d = cfg.hidden, cfg.head_dim
    h1 = layernorm(xf, params["ln1_g"], params["ln1_b"]).astype(np.float16)
    qkv = gemm(h1, packed["w_qkv"], params["b_qkv"])
    q = (qkv[:, :h] * (float(d) ** -0.5)).astype(np.float16)
    k = qkv[:, h:2 * h].astype(np.float16)
    v = qkv[:, 2 * h:].astype(np.float16)
    return h1, q, k, v, qkv[:, h:2 * h], qkv[:, 2 * h:]


def _after_attention(xf, o, params, packed):
    """Output projection with residual, LN2, FFN with residual for rows xf [M, h]
    and their attention output o (fp16).  Returns x1_64, x1, h2, f, y64."""
    x1_64 = xf.astype(np.float64) + gemm(o, packed["w_out"], params["b_out"])
    x1 = x1_64.astype(np.float16)
    h2 = layernorm(x1, params["ln2_g"], params["ln2_b"]).astype(np.float16)
    f = np.maximum(gemm(h2, packed["w_fc1"], params["b_fc1"]), 0.0).astype(np.float16)
    y64 = x1.astype(np.float64) + gemm(f, packed["w_fc2"], params["b_fc2"])
    return x1_64, x1, h2, f, y64


def layer_step(x16: np.ndarray, params: dict, packed: dict, cache: dict, cfg: LayerConfig,
               pos: int, want: tuple = ()) -> dict:
    """One pre-LN decoder layer over T new tokens per sequence at positions pos..pos+T-1.

    x16 fp16 [B, T, h].  Appends the new K/V to `cache`.  Returns {"y": fp16 [B, T, h],
    "y64": float64 [B, T, h] before the final rounding, plus any names in `want`}."""
    B, T, h = x16.shape
    H, d = cfg.heads, cfg.head_dim
    r = {}
    xf = x16.reshape(B * T, h)
    h1, q, k, v, k64, v64 = _qkv(xf, params, packed, cfg)
    to_bhtd = lambda a: a.reshape(B, T, H, d).transpose(0, 2, 1, 3)
    _cache_append(cache, cfg, to_bhtd(k), to_bhtd(v), pos)
    o64 = _attend(to_bhtd(q), cache, cfg, pos)                 # [B, H, T, d]
    o = o64.transpose(0, 2, 1, 3).reshape(B * T, h).astype(np.float16)
    x1_64, x1, h2, f, y64 = _after_attention(xf, o, params, packed)
    r["y"] = y64.astype(np.float16).reshape(B, T, h)
    r["y64"] = y64.reshape(B, T, h)
    local = {"h1": h1, "q": q, "k": k, "v": v, "k64": k64, "v64": v64,
             "o": o, "o64": o64, "x1": x1, "x1_64": x1_64,
             "h2": h2, "f": f}
    for name in want:
        r[name] = local[name]
    return r


def cache_fill(cache: dict, cfg: LayerConfig, k16: np.ndarray, v16: np.ndarray, pos: int = 0) -> None:
    """Put given fp16 K/V of tokens at positions pos..pos+T-1 into the cache, quantised
    exactly as the layer appends its own (teacher forcing: K/V computed elsewhere).
    k16, v16 [B, T, h]."""
    B, T, h = k16.shape
    H, d = cfg.heads, cfg.head_dim
    to_bhtd = lambda a: np.ascontiguousarray(np.asarray(a, np.float16).reshape(B, T, H, d).transpose(0, 2, 1, 3))
    _cache_append(cache, cfg, to_bhtd(k16), to_bhtd(v16), pos)


def layer_rows(x16: np.ndarray, positions, params: dict, packed: dict, cache: dict, cfg: LayerConfig,
               want: tuple = ()) -> dict:
    """The layer applied to given rows under teacher forcing: row r of every sequence
    is the token at position positions[r], and its query attends over cache positions
    0..positions[r], which the cache must already hold (cache_fill).  Nothing is
    appended.  The arithmetic is layer_step's; the row's own K/V are returned (for
    comparison with those in the cache) but not used.

    x16 fp16 [B, R, h].  Returns {"y", "y64"} [B, R, h] plus any names in `want`."""
    B, R, h = x16.shape
    H, d = cfg.heads, cfg.head_dim
    positions = np.asarray(positions, np.int64)
    assert positions.shape == (R,)
    xf = x16.reshape(B * R, h)
    h1, q, k, v, k64, v64 = _qkv(xf, params, packed, cfg)
    qb = q.reshape(B, R, H, d).transpose(0, 2, 1, 3)           # [B, H, R, d]
    n = int(positions.max()) + 1
    mask = np.arange(n)[None, :] > positions[:, None]          # [R, n]
    o64 = np.empty((B, H, R, d), np.float64)
    for b in range(B):
        kk, vv = _cache_read(cache, cfg, n, b)                 # [H, n, d]
        sc = qb[b].astype(np.float64) @ np.swapaxes(kk, -1, -2)  # [H, R, n]
        sc[:, mask] = -np.inf
        o64[b] = softmax(sc, axis=-1) @ vv
    o = o64.transpose(0, 2, 1, 3).reshape(B * R, h).astype(np.float16)
    x1_64, x1, h2, f, y64 = _after_attention(xf, o, params, packed)
    r = {"y": y64.astype(np.float16).reshape(B, R, h), "y64": y64.reshape(B, R, h)}
    rows = lambda a: a.reshape(B, R, -1)
    local = {"h1": rows(h1), "q": rows(q), "k": rows(k), "v": rows(v), "k64": rows(k64), "v64": rows(v64),
             "o": rows(o), "o64": o64, "x1": rows(x1), "x1_64": rows(x1_64), "h2": rows(h2), "f": rows(f)}
    for name in want:
        r[name] = local[name]
    return r


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Greedy choice per row; ties go to the lowest token id (np.argmax returns the first max)."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def embed(ids: np.ndarray, emb16: np.ndarray, pos16: np.ndarray, pos0: int) -> np.ndarray:
    """x = (E[id] + Pos[p + 2])[16] for token ids [B, T] at positions pos0..pos0+T-1."""
    T = ids.shape[1]
    p = np.arange(pos0, pos0 + T) + 2
    return (emb16[ids].astype(np.float64) + pos16[p][None].astype(np.float64)).astype(np.float16)


def lm_head_logits(x16: np.ndarray, lnf_g, lnf_b, emb16) -> np.ndarray:
    """Final LayerNorm ([16]) then logits = LN(x) E^T in float64; x16 [B, h] -> [B, V]."""
    xf = layernorm(x16, lnf_g, lnf_b).astype(np.float16)
    return xf.astype(np.float64) @ emb16.astype(np.float64).T


def model_params(seed: int, mcfg: ModelConfig, bias_sigma: float = 0.0) -> dict:
    """Embedding, positions and final-LN parameters from the seeded generator."""
    h = mcfg.layer.hidden
    p = {"embed": synth.normal_f16(seed, synth.STREAM["embed"], (mcfg.vocab, h), 0.02),
         "pos": synth.normal_f16(seed, synth.STREAM["pos"], (mcfg.max_pos, h), 0.02)}
    if bias_sigma > 0:
        p["lnf_g"] = synth.normal_f16(seed, synth.STREAM["lnf_g"], (h,), 1.0)
        p["lnf_b"] = synth.normal_f16(seed, synth.STREAM["lnf_b"], (h,), bias_sigma)
    else:
        p["lnf_g"] = np.ones(h, np.float16)
        p["lnf_b"] = np.zeros(h, np.float16)
    return p


def generate(prompt_ids: np.ndarray, gen_len: int, seed: int, mcfg: ModelConfig,
             bias_sigma: float = 0.0, layers_params=None) -> dict:
    """Greedy generation: prefill of the prompt yields token 1, each of gen_len-1 decode
    steps yields one more.  Returns {"tokens": int32 [B, gen_len], "logits": list of
    float64 [B, V] per generated token}."""
    cfg = mcfg.layer
    B, P = prompt_ids.shape
    mp = model_params(seed, mcfg, bias_sigma)
    if layers_params is None:
        layers_params = [layer_params(seed, cfg, l, bias_sigma) for l in range(mcfg.layers)]
    packed = [pack_layer(p, cfg) for p in layers_params]
    caches = [new_cache(cfg, B, P + gen_len) for _ in range(mcfg.layers)]
    tokens = np.zeros((B, gen_len), np.int32)
    logits_all = []
    x = embed(prompt_ids, mp["embed"], mp["pos"], 0)
    pos = 0
    for step in range(gen_len):
        for l in range(mcfg.layers):
            x = layer_step(x, layers_params[l], packed[l], caches[l], cfg, pos)["y"]
        logits = lm_head_logits(x[:, -1], mp["lnf_g"], mp["lnf_b"], mp["embed"])
        logits_all.append(logits)
        tok = argmax_lowest(logits)
        tokens[:, step] = tok
        pos += x.shape[1]
        if step + 1 < gen_len:
            x = embed(tok[:, None], mp["embed"], mp["pos"], pos)
    return {"tokens": tokens, "logits": logits_all}
