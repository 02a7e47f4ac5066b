"""fq_generate (embedding, prefill, decode steps, LM head, greedy argmax) on
a small random-init model against the oracle's generation, and layer
streaming from pinned host memory against resident weights."""
import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import LayerConfig, ModelConfig
from tests._util import dev, host, assert_close, log

pytestmark = pytest.mark.gpu
fq = pytest.importorskip("bit_weight_kv_amd")

H, NH, F, V = 256, 4, 1024, 512


def _gpu_generate(L, B, P, G, seed, **model_kw):
    model = fq.Model(H, NH, F, L, vocab=V, max_pos=P + G + 2, **model_kw)
    model.init_random(seed)
    kv = fq.KVCache(model, B, P + G)
    ids = synth.token_ids(seed, synth.STREAM["prompt"], (B, P), V)
    logits = torch.empty((G, B, V), dtype=torch.float32, device="cuda:0")
    out, st = fq.fq_generate(model, kv, ids, G, logits=logits)
    lg = host(logits)
    kv.close()
    model.close()
    return ids, out, lg, st


# Logits come after every layer plus the final LayerNorm: the per-layer bound
# (relative L2 5e-3) is allowed to compound once more over the stack.
LOGIT_REL_L2 = 1e-2


def _compare(out, lg, ref, what):
    """Logits within tolerance while the token streams agree; a disagreement is
    allowed only at a near-tie of the oracle's logits, and ends the comparison."""
    B, G = out.shape
    for b in range(B):
        for t in range(G):
            r, m = assert_close(lg[t, b], ref["logits"][t][b], rel=LOGIT_REL_L2, abs_=3e-2,
                                what=f"{what} logits b={b} t={t}")
            if t == 0 and b == 0:
                log(f"{what}: logits rel_l2 {r:.2e} max_abs {m:.2e}")
            if out[b, t] != ref["tokens"][b, t]:
                r = ref["logits"][t][b]
                gap = abs(r[out[b, t]] - r[ref["tokens"][b, t]])
                assert gap < 2e-2, f"{what}: token mismatch b={b} t={t} with logit gap {gap}"
                break


def test_generate_matches_oracle():
    L, B, P, G = 2, 4, 16, 6
    log("generate small model")
    ids, out, lg, st = _gpu_generate(L, B, P, G, seed=0)
    mcfg = ModelConfig(LayerConfig(H, NH, F), L, V, P + G + 2)
    ref = oracle.generate(ids, G, 0, mcfg)
    _compare(out, lg, ref, "resident 4-bit")
    assert st.tokens_per_s > 0 and st.prefill_s > 0 and st.decode_s > 0
    assert abs(st.tokens_per_s - B * G / (st.prefill_s + st.decode_s)) < 1e-6 * st.tokens_per_s


@pytest.mark.parametrize("weight,cache", [(True, False), (False, False)])
def test_generate_compression_toggles_match_oracle(weight, cache):
    """Weight-only compression (fp16 KV cache) and no compression, against the
    oracle's generation with the same switches."""
    L, B, P, G = 2, 4, 16, 6
    log(f"generate compress_weight={weight} compress_cache={cache}")
    ids, out, lg, st = _gpu_generate(L, B, P, G, seed=4, compress_weight=weight, compress_cache=cache)
    mcfg = ModelConfig(LayerConfig(H, NH, F, compress_weight=weight, compress_cache=cache), L, V, P + G + 2)
    ref = oracle.generate(ids, G, 4, mcfg)
    _compare(out, lg, ref, f"weight={weight} cache={cache}")


@pytest.mark.parametrize("cache", [True, False])
def test_offloaded_cache_equals_resident(cache):
    """KV cache of layers beyond cache_resident_layers in pinned host memory
    (staged prefix in, new positions back, per pass): identical tokens and
    logits to the all-resident cache, with and without prefetch overlap and
    together with streamed weights; the copied byte counts are the prefix and
    new-position volumes."""
    L, B, P, G = 4, 3, 12, 5
    log(f"offloaded cache compress_cache={cache}")
    ids, a_out, a_lg, _ = _gpu_generate(L, B, P, G, seed=5, compress_cache=cache)
    runs = [_gpu_generate(L, B, P, G, seed=5, compress_cache=cache, cache_resident_layers=1),
            _gpu_generate(L, B, P, G, seed=5, compress_cache=cache, cache_resident_layers=0, overlap=False),
            _gpu_generate(L, B, P, G, seed=5, compress_cache=cache, cache_resident_layers=2, resident_layers=1)]
    for _, out, lg, _ in runs:
        assert np.array_equal(out, a_out) and np.array_equal(lg, a_lg)
    d = H // NH
    per_pos = B * NH * (2 * (d // 2 + d // 64 * 4) if cache else 2 * d * 2)  # one position, all sequences, K and V
    h2d_pos = (G - 1) * P + (G - 2) * (G - 1) // 2                        # decode pass at pos stages [0, pos)
    d2h_pos = P + G - 1                                                    # every position written back once
    for (_, _, _, st), off in zip(runs, (L - 1, L, L - 2)):
        assert st.kv_h2d_bytes == off * per_pos * h2d_pos and st.kv_d2h_bytes == off * per_pos * d2h_pos
    mcfg = ModelConfig(LayerConfig(H, NH, F, compress_cache=cache), L, V, P + G + 2)
    _compare(runs[0][1], runs[0][2], oracle.generate(ids, G, 5, mcfg), f"offloaded cache={cache}")
    # prefill in chunks of 2 sequences (max_tokens = 2 prompts): one staging and
    # one write-back per layer serve every chunk
    _, r_out, r_lg, _ = _gpu_generate(L, B, P, G, seed=5, compress_cache=cache, max_tokens=2 * P)
    _, o_out, o_lg, _ = _gpu_generate(L, B, P, G, seed=5, compress_cache=cache, max_tokens=2 * P,
                                      cache_resident_layers=1)
    assert np.array_equal(o_out, r_out) and np.array_equal(o_lg, r_lg)


def test_generate_deterministic_and_batch_independent():
    L, B, P, G = 2, 3, 12, 4
    ids, out1, lg1, _ = _gpu_generate(L, B, P, G, seed=1)
    _, out2, lg2, _ = _gpu_generate(L, B, P, G, seed=1)
    assert np.array_equal(out1, out2) and np.array_equal(lg1, lg2)


def test_streamed_fp16_weights_equal_resident():
    """fp16 weights: all resident vs. layers 1..3 streamed from pinned host
    memory with overlap, vs. streamed without overlap: identical results."""
    L, B, P, G = 4, 2, 10, 4
    log("streaming equivalence")
    _, a_out, a_lg, a_st = _gpu_generate(L, B, P, G, seed=2, compress_weight=False)
    _, b_out, b_lg, b_st = _gpu_generate(L, B, P, G, seed=2, compress_weight=False, resident_layers=1)
    _, c_out, c_lg, c_st = _gpu_generate(L, B, P, G, seed=2, compress_weight=False, resident_layers=1, overlap=False)
    assert np.array_equal(a_out, b_out) and np.array_equal(a_lg, b_lg)
    assert np.array_equal(a_out, c_out) and np.array_equal(a_lg, c_lg)
    layer_bytes = (4 * H * H + 2 * H * F) * 2
    assert a_st.h2d_bytes == 0
    # streamed layers 1, 2, 3 use staging slots 1, 0, 1: the first pass copies all
    # three, later passes find layer 2 still staged in slot 0 and copy two
    assert b_st.h2d_bytes == (3 + 2 * (G - 1)) * layer_bytes and b_st.h2d_s > 0


def test_streamed_shared_host_blobs_match_oracle():
    """4 layers all streamed from 2 host blobs: layer l holds the weights generated
    for layer l % 2; the oracle runs the same tied-weight fp16 model."""
    L, B, P, G = 4, 2, 8, 4
    ids, out, lg, st = _gpu_generate(L, B, P, G, seed=3, compress_weight=False, resident_layers=0, host_layers=2)
    cfg = LayerConfig(H, NH, F, compress_weight=False)
    mcfg = ModelConfig(cfg, L, V, P + G + 2)
    lps = [oracle.layer_params(3, cfg, l % 2) for l in range(L)]
    ref = oracle.generate(ids, G, 3, mcfg, layers_params=lps)
    _compare(out, lg, ref, "streamed fp16")


def test_streamed_packed_weights_equal_resident():
    """4-bit weights: all resident vs. layers 1..3 streamed in packed form
    (codes + {min, scale}, 0.5625 byte per weight) from pinned host memory,
    with and without overlap: identical tokens and logits."""
    L, B, P, G = 4, 2, 10, 4
    log("packed streaming equivalence")
    _, a_out, a_lg, a_st = _gpu_generate(L, B, P, G, seed=2)
    _, b_out, b_lg, b_st = _gpu_generate(L, B, P, G, seed=2, resident_layers=1)
    _, c_out, c_lg, c_st = _gpu_generate(L, B, P, G, seed=2, resident_layers=1, overlap=False)
    assert np.array_equal(a_out, b_out) and np.array_equal(a_lg, b_lg)
    assert np.array_equal(a_out, c_out) and np.array_equal(a_lg, c_lg)
    elems = 4 * H * H + 2 * H * F
    layer_bytes = elems // 2 + elems // 64 * 4
    assert a_st.h2d_bytes == 0
    assert b_st.h2d_bytes == (3 + 2 * (G - 1)) * layer_bytes and b_st.h2d_s > 0


def test_streamed_packed_shared_host_blobs_match_oracle():
    """4 layers of 4-bit weights all streamed from 2 packed host blobs: layer l
    holds the weights generated for layer l % 2; the oracle runs the same
    tied-weight model."""
    L, B, P, G = 4, 2, 8, 4
    ids, out, lg, st = _gpu_generate(L, B, P, G, seed=4, resident_layers=0, host_layers=2)
    cfg = LayerConfig(H, NH, F)
    mcfg = ModelConfig(cfg, L, V, P + G + 2)
    lps = [oracle.layer_params(4, cfg, l % 2) for l in range(L)]
    ref = oracle.generate(ids, G, 4, mcfg, layers_params=lps)
    _compare(out, lg, ref, "streamed 4-bit")


def test_packed_weight_of_streamed_layer_is_rejected():
    model = fq.Model(H, NH, F, 2, vocab=V, max_pos=16, resident_layers=1)
    try:
        model.packed_weight(0, 0)
        with pytest.raises(fq.FqError):
            model.packed_weight(1, 0)
    finally:
        model.close()


def test_progress_callback_reports_every_token_in_order():
    L, B, P, G = 2, 2, 8, 5
    seen = []
    fq.fq_set_progress(lambda done, total: seen.append((done, total)))
    try:
        ids, out, lg, _ = _gpu_generate(L, B, P, G, seed=3)
    finally:
        fq.fq_set_progress(None)
    assert seen == [(t, G) for t in range(1, G + 1)]
    # the report changes nothing: same tokens and logits without it
    _, out2, lg2, _ = _gpu_generate(L, B, P, G, seed=3)
    assert np.array_equal(out, out2) and np.array_equal(lg, lg2)


@pytest.mark.parametrize("compress", [True, False])
@pytest.mark.parametrize("replace", [1, 2])
def test_replaced_streamed_layer_is_copied_again(compress, replace):
    """Layers 1 and 2 streamed (staging slots 1 and 0).  After a generation the
    slots still hold those layers; replacing one of them with fq_model_set_layer
    must make the next generation copy the new weights in: its tokens and
    logits equal those of an all-resident model holding the same weights."""
    L, B, P, G = 3, 2, 10, 4
    names = ("w_qkv", "w_out", "w_fc1", "w_fc2", "b_qkv", "b_out", "b_fc1", "b_fc2",
             "ln1_g", "ln1_b", "ln2_g", "ln2_b")
    new = oracle.layer_params(9, LayerConfig(H, NH, F), replace, bias_sigma=0.02)
    new_dev = {n: dev(new[n]) for n in names}
    ids = synth.token_ids(6, synth.STREAM["prompt"], (B, P), V)
    results = []
    for resident in (1, -1):
        model = fq.Model(H, NH, F, L, vocab=V, max_pos=P + G + 2, compress_weight=compress,
                         resident_layers=resident)
        model.init_random(6)
        kv = fq.KVCache(model, B, P + G)
        if resident == 1:
            fq.fq_generate(model, kv, ids, G)  # leaves layers 1 and 2 in the staging slots
        model.set_layer(replace, new_dev)
        torch.cuda.synchronize()
        logits = torch.empty((G, B, V), dtype=torch.float32, device="cuda:0")
        out, _ = fq.fq_generate(model, kv, ids, G, logits=logits)
        results.append((out, host(logits)))
        kv.close()
        model.close()
    (s_out, s_lg), (r_out, r_lg) = results
    assert np.array_equal(s_out, r_out) and np.array_equal(s_lg, r_lg)
