"""Group-wise 4-bit min/max (asymmetric) quantisation: the encoding itself.

Source: FlexGen README (giters.com mirror), "Extreme Compression" (weights and
attention cache go to 4 bits); inference/research record, "Mechanism" (4-bit
so that more state fits on the GPU).  The pages state only "4 bits"; this
oracle takes the plainest min/max reading with a fixed group of 64:

  per group of 64 consecutive values v (fp16, widened exactly to fp32):
    mn  = min v   (a -0 minimum is stored as +0)
    mx  = max v
    s32 = (mx - mn) / 15            fp32 subtract, fp32 divide, both RNE
                                    (a zero scale is stored as +0)
    s16 = fp16(s32) (RNE);  s = fp32(s16)
    code_i = 0                                      if s == 0
           = clamp(rint_half_even((v_i - mn) / s), 0, 15)   otherwise
    stored: codes as nibbles (element 2k in the low nibble of byte k),
            meta = fp16 pair {mn, s16} per group.
  dequantised value: mn + code * s (exact), rounded to fp16 for GEMM operands.

Pinned in tests/test_oracle_quant.py against worked examples (tests/golden/),
brute force over the 16 levels, the round-trip bound s/2, and the ~70 %
memory saving the README states for --compress-weight.
"""
import numpy as np

GROUP = 64


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [..., n] (n even, values 0..15) -> bytes [..., n/2]; even element in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """bytes [..., n/2] -> codes [..., n]."""
    p = packed.astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def quantize(x16: np.ndarray, group: int = GROUP):
    """fp16 array [..., cols] -> (codes uint8 [..., cols/2], meta fp16 [..., cols/group, 2]).

    Groups are `group` consecutive elements along the last axis."""
    x16 = np.asarray(x16)
    assert x16.dtype == np.float16, "quantize takes fp16 input"
    cols = x16.shape[-1]
    assert cols % group == 0 and group % 2 == 0
    ng = cols // group
    v = x16.astype(np.float32).reshape(x16.shape[:-1] + (ng, group))
    mn = v.min(axis=-1)
    mx = v.max(axis=-1)
    mn = np.where(mn == np.float32(0), np.float32(0), mn).astype(np.float32)   # canonical +0
    s32 = (mx - mn) / np.float32(15.0)
    s32 = np.where(s32 == np.float32(0), np.float32(0), s32).astype(np.float32)  # canonical +0 scale
    s16 = s32.astype(np.float16)
    s = s16.astype(np.float32)
    zero = (s == np.float32(0))
    safe = np.where(zero, np.float32(1), s)
    with np.errstate(invalid="ignore"):
        q = (v - mn[..., None]) / safe[..., None]
    codes = np.clip(np.rint(q), 0, 15)
    codes = np.where(zero[..., None], 0, codes).astype(np.uint8)
    codes = codes.reshape(x16.shape)
    meta = np.stack([mn.astype(np.float16), s16], axis=-1)
    return pack_nibbles(codes), meta


def _levels(codes_packed, meta, group):
    codes = unpack_nibbles(codes_packed).astype(np.float64)
    cols = codes.shape[-1]
    ng = cols // group
    c = codes.reshape(codes.shape[:-1] + (ng, group))
    mn = meta[..., 0].astype(np.float64)[..., None]
    s = meta[..., 1].astype(np.float64)[..., None]
    return (mn + c * s).reshape(codes.shape)


def dequant_f64(codes_packed: np.ndarray, meta: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Exact reconstruction mn + code*s in float64 (the product of an fp16 scale and a
    code below 16 and its sum with an fp16 minimum are exact in float64)."""
    return _levels(codes_packed, meta, group)


def dequant_f16(codes_packed: np.ndarray, meta: np.ndarray, group: int = GROUP) -> np.ndarray:
    """fp16(mn + code*s) with one round-to-nearest-even: the GEMM operand."""
    return _levels(codes_packed, meta, group).astype(np.float16)
