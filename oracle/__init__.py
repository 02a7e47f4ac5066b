"""CPU oracle for the 4-bit weight + 4-bit KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the GPU library computes, used to check it.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the product path (the HIP library and its Python binding) never
does, and shares no code with it.

Pages followed (FlexGen, Sheng et al., "High-Throughput Generative Inference
of Large Language Models with a Single GPU"):
  * FlexGen README (giters.com mirror), key features, "Extreme Compression":
    weights and the attention cache are compressed to 4 bits.
  * same page, "Handle Out-of-memory": --compress-weight cuts weight memory by
    about 70 %.
  * same page, "Benchmark Results", Metric bullet: generation throughput =
    generated tokens / (prompt time + generation time).
  * pith.science record of the paper, abstract: 4-bit weights and cache,
    effective batch 144 on OPT-175B.
  * inference/research record of the paper, "Mechanism" field: weights and
    the attention cache are compressed to 4 bits so that more state fits on
    the GPU.
The pages fix neither group size, grouping axis, min/max versus symmetric
ranges, scale precision nor rounding; the readings taken here (group 64 along
the contiguous axis, unsigned codes offset by the group minimum, fp16
min/scale, IEEE fp32 arithmetic with round-half-to-even) are listed with the
rest in the design notes and are shared with the GPU library by specification
only.

Floating point: quantisation decisions are taken in IEEE fp32 (the precision
the GPU kernel uses for them); every other operation runs in float64 with
fp16 rounding only at the storage points of the layer (see model.py).
"""
from .quant import quantize, dequant_f16, dequant_f64, pack_nibbles, unpack_nibbles, GROUP
from .ops import gemm, layernorm, attention_decode, attention_prefill_causal, softmax
from .model import (LayerConfig, ModelConfig, layer_params, pack_layer, new_cache, layer_step,
                    layer_rows, cache_fill, generate, embed, lm_head_logits, argmax_lowest)

__all__ = [
    "quantize", "dequant_f16", "dequant_f64", "pack_nibbles", "unpack_nibbles", "GROUP",
    "gemm", "layernorm", "attention_decode", "attention_prefill_causal", "softmax",
    "LayerConfig", "ModelConfig", "layer_params", "pack_layer", "new_cache", "layer_step",
    "layer_rows", "cache_fill",
    "generate", "embed", "lm_head_logits", "argmax_lowest",
]
