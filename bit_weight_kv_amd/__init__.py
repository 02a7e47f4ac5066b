"""Python binding of libfq (4-bit weight + 4-bit KV-cache decoding on MI355X).

Argument marshalling only: every function here forwards to the C ABI in
include/fq.h with the same name.  Device buffers are torch tensors on the
current HIP device (torch supplies memory and streams); every step of the
computation runs in the HIP kernels of libfq.so.  A missing library raises
at import time -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libfq.so is not built ({LIB_PATH}); run python bit_weight_kv_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_u32, c_u64, c_f32, c_f64, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64,
                                                  ctypes.c_float, ctypes.c_double, ctypes.c_void_p)

FQ_OK, FQ_ERR_INVALID, FQ_ERR_UNSUPPORTED, FQ_ERR_OOM, FQ_ERR_HIP = 0, -1, -2, -3, -4
FQ_GROUP = 64
FQ_WEIGHT_PACKED4, FQ_WEIGHT_F16 = 0, 1
FQ_EPI_BIAS, FQ_EPI_QSCALE, FQ_EPI_RELU, FQ_EPI_RESIDUAL, FQ_EPI_F32OUT = 1, 2, 4, 8, 16


class FqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libfq status {status}: {msg}")
        self.status = status


class fq_packed(ctypes.Structure):
    _fields_ = [("codes", c_vp), ("meta", c_vp), ("rows", c_i64), ("cols", c_i64), ("group", c_i32)]


class fq_weight(ctypes.Structure):
    _fields_ = [("kind", c_i32), ("packed", fq_packed), ("w16", c_vp), ("n", c_i64), ("k", c_i64)]


class fq_kv_layer(ctypes.Structure):
    _fields_ = [("k_codes", c_vp), ("k_meta", c_vp), ("v_codes", c_vp), ("v_meta", c_vp), ("batch", c_i64),
                ("heads", c_i32), ("head_dim", c_i32), ("capacity", c_i64), ("group", c_i32), ("bits", c_i32),
                ("k16", c_vp), ("v16", c_vp)]


class fq_model_config(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("heads", c_i32), ("ffn", c_i32), ("layers", c_i32), ("vocab", c_i32),
                ("max_pos", c_i32)]


class fq_policy(ctypes.Structure):
    _fields_ = [("compress_weight", c_i32), ("compress_cache", c_i32), ("resident_layers", c_i32),
                ("host_layers", c_i32), ("overlap", c_i32), ("max_tokens", c_i64), ("cache_resident_layers", c_i32)]


class fq_layer_weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("w_qkv", "w_out", "w_fc1", "w_fc2", "b_qkv", "b_out", "b_fc1", "b_fc2",
                                    "ln1_g", "ln1_b", "ln2_g", "ln2_b")]


class fq_capture(ctypes.Structure):
    _fields_ = [("layer", c_i32), ("b0", c_i64), ("nb", c_i64), ("capacity", c_i64), ("x_in", c_vp),
                ("y_out", c_vp), ("k16", c_vp), ("v16", c_vp), ("x1", c_vp)]


class fq_kernel_stats(ctypes.Structure):
    _fields_ = [("launches", c_i64), ("seconds", c_f64), ("flops", c_f64), ("bytes", c_f64), ("dropped", c_i64)]


KERNEL_CLASSES = ("gemm_prefill", "gemm_decode", "lm_head", "decode_attention", "prefill_attention", "kv_append",
                  "quantize", "layernorm")


class fq_gen_stats(ctypes.Structure):
    _fields_ = [("prefill_s", c_f64), ("decode_s", c_f64), ("tokens_per_s", c_f64), ("h2d_bytes", c_f64),
                ("h2d_s", c_f64), ("kv_h2d_bytes", c_f64), ("kv_d2h_bytes", c_f64)]


_P = ctypes.POINTER
_SIGS = {
    "fq_last_error": (ctypes.c_char_p, []),
    "fq_version": (ctypes.c_char_p, []),
    "fq_quantize": (c_i32, [c_vp, c_i64, c_i64, c_i64, _P(fq_packed), c_vp]),
    "fq_dequantize": (c_i32, [_P(fq_packed), c_vp, c_vp]),
    "fq_dequant_gemm": (c_i32, [c_vp, c_i64, c_i64, _P(fq_weight), c_vp, c_vp, c_i64, c_u32, c_f32, c_i64, c_vp,
                                c_i64, c_vp]),
    "fq_dequant_gemm_noalloc": (c_i32, [c_vp, c_i64, c_i64, _P(fq_weight), c_vp, c_vp, c_i64, c_u32, c_f32, c_i64,
                                        c_vp, c_i64, c_vp]),
    "fq_kv_append": (c_i32, [_P(fq_kv_layer), c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp]),
    "fq_decode_attention": (c_i32, [c_vp, c_i64, _P(fq_kv_layer), c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "fq_prefill_attention": (c_i32, [c_vp, c_i64, _P(fq_kv_layer), c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "fq_qkv_gemm_append": (c_i32, [c_vp, c_i64, c_i64, _P(fq_weight), c_vp, c_f32, _P(fq_kv_layer), c_i64, c_i64,
                                   c_i64, c_i64, c_vp, c_i64, c_vp]),
    "fq_layernorm": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_f32, c_vp, c_i64, c_vp]),
    "fq_model_create": (c_i32, [_P(fq_model_config), _P(fq_policy), _P(c_vp)]),
    "fq_model_destroy": (c_i32, [c_vp]),
    "fq_model_set_layer": (c_i32, [c_vp, c_i32, _P(fq_layer_weights), c_vp]),
    "fq_model_set_embeddings": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "fq_model_init_random": (c_i32, [c_vp, c_u64, c_f64, c_vp]),
    "fq_model_packed_weight": (c_i32, [c_vp, c_i32, c_i32, _P(fq_packed)]),
    "fq_model_set_capture": (c_i32, [c_vp, _P(fq_capture), c_i32]),
    "fq_kv_create": (c_i32, [c_vp, c_i64, c_i64, _P(c_vp)]),
    "fq_kv_destroy": (c_i32, [c_vp]),
    "fq_kv_layer_view": (c_i32, [c_vp, c_i32, _P(fq_kv_layer)]),
    "fq_layer_step": (c_i32, [c_vp, c_i32, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "fq_generate": (c_i32, [c_vp, c_vp, _P(c_i32), c_i64, c_i64, c_i64, _P(c_i32), c_vp, _P(fq_gen_stats), c_vp]),
    "fq_synth_normal_f16": (c_i32, [c_vp, c_i64, c_u64, c_u64, c_i64, c_f64, c_vp]),
    "fq_synth_token_ids": (c_i32, [c_vp, c_i64, c_u64, c_u64, c_i32, c_vp]),
    "fq_set_progress": (None, [c_vp, c_vp]),
    "fq_timing_start": (c_i32, [c_u32]),
    "fq_timing_stop": (c_i32, [_P(fq_kernel_stats)]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def fq_last_error() -> str:
    return _lib.fq_last_error().decode()


def fq_version() -> str:
    return _lib.fq_version().decode()


def _check(status):
    if status != FQ_OK:
        raise FqError(status, fq_last_error())


def _ptr(t):
    return None if t is None else c_vp(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_vp(stream.cuda_stream)


def _keep(struct, *tensors):
    """Tie the tensors' lifetime to the ctypes struct that holds their raw pointers."""
    struct._keep = tensors
    return struct


def packed_view(codes, meta, rows, cols):
    """fq_packed over torch tensors codes uint8 [rows, cols/2], meta int16 [rows, cols/64, 2]."""
    return _keep(fq_packed(c_vp(codes.data_ptr()), c_vp(meta.data_ptr()), rows, cols, FQ_GROUP), codes, meta)


def fq_quantize(x, codes, meta, stream=None):
    """x fp16 [rows, cols] (row stride x.stride(0)) -> codes uint8 [rows, cols/2], meta int16 [rows, cols/64, 2]."""
    rows, cols = x.shape
    p = packed_view(codes, meta, rows, cols)
    _check(_lib.fq_quantize(_ptr(x), rows, cols, x.stride(0), ctypes.byref(p), _stream(stream)))


def fq_dequantize(codes, meta, rows, cols, y, stream=None):
    p = packed_view(codes, meta, rows, cols)
    _check(_lib.fq_dequantize(ctypes.byref(p), _ptr(y), _stream(stream)))


def weight_packed(codes, meta, n, k):
    return _keep(fq_weight(FQ_WEIGHT_PACKED4, packed_view(codes, meta, n, k), None, n, k), codes, meta)


def weight_f16(w):
    n, k = w.shape
    return _keep(fq_weight(FQ_WEIGHT_F16, fq_packed(), c_vp(w.data_ptr()), n, k), w)


def fq_dequant_gemm(A, W, C, bias=None, residual=None, epilogue=0, qscale=1.0, qscale_cols=0, stream=None):
    """C = epilogue(A @ W^T).  A fp16 [M, K]; W an fq_weight; C fp16/fp32 [M, N]."""
    M = A.shape[0]
    ldr = residual.stride(0) if residual is not None else 0
    _check(_lib.fq_dequant_gemm(_ptr(A), M, A.stride(0), ctypes.byref(W), _ptr(bias), _ptr(residual), ldr,
                                epilogue, qscale, qscale_cols, _ptr(C), C.stride(0), _stream(stream)))


def fq_dequant_gemm_noalloc(A, W, C, bias=None, residual=None, epilogue=0, qscale=1.0, qscale_cols=0, stream=None):
    """fq_dequant_gemm without any device allocation (split-K partials in the library's fixed scratch)."""
    M = A.shape[0]
    ldr = residual.stride(0) if residual is not None else 0
    _check(_lib.fq_dequant_gemm_noalloc(_ptr(A), M, A.stride(0), ctypes.byref(W), _ptr(bias), _ptr(residual), ldr,
                                        epilogue, qscale, qscale_cols, _ptr(C), C.stride(0), _stream(stream)))


def kv_layer_view(k_codes, k_meta, v_codes, v_meta):
    """fq_kv_layer over torch tensors: codes uint8 [B, H, S, d/2], meta int16 [B, H, S, d/64, 2]."""
    B, H, S, half = k_codes.shape
    v = fq_kv_layer(c_vp(k_codes.data_ptr()), c_vp(k_meta.data_ptr()), c_vp(v_codes.data_ptr()),
                    c_vp(v_meta.data_ptr()), B, H, half * 2, S, FQ_GROUP, 4, None, None)
    return _keep(v, k_codes, k_meta, v_codes, v_meta)


def kv_layer_view_f16(k16, v16):
    """fq_kv_layer (bits 16) over torch fp16 tensors k16, v16 [B, H, S, d]."""
    B, H, S, d = k16.shape
    v = fq_kv_layer(None, None, None, None, B, H, d, S, FQ_GROUP, 16, c_vp(k16.data_ptr()), c_vp(v16.data_ptr()))
    return _keep(v, k16, v16)


def fq_kv_append(kv, k, v, ld, b0, B, T, pos, stream=None):
    _check(_lib.fq_kv_append(ctypes.byref(kv), _ptr(k) if isinstance(k, torch.Tensor) else c_vp(k),
                             _ptr(v) if isinstance(v, torch.Tensor) else c_vp(v), ld, b0, B, T, pos,
                             _stream(stream)))


def fq_qkv_gemm_append(A, W, bias, qscale, kv, b0, B, T, pos, C, stream=None):
    """QKV projection (+bias, q scaled) with the K/V append fused: q -> C[:, :h], K/V -> cache."""
    _check(_lib.fq_qkv_gemm_append(_ptr(A), A.shape[0], A.stride(0), ctypes.byref(W), _ptr(bias), qscale,
                                   ctypes.byref(kv), b0, B, T, pos, _ptr(C), C.stride(0), _stream(stream)))


def fq_decode_attention(q, kv, b0, B, length, out, ldq=None, ldo=None, stream=None):
    _check(_lib.fq_decode_attention(_ptr(q), ldq or q.stride(0), ctypes.byref(kv), b0, B, length, _ptr(out),
                                    ldo or out.stride(0), _stream(stream)))


def fq_prefill_attention(q, kv, b0, B, T, pos, out, ldq=None, ldo=None, stream=None):
    _check(_lib.fq_prefill_attention(_ptr(q), ldq or q.stride(0), ctypes.byref(kv), b0, B, T, pos, _ptr(out),
                                     ldo or out.stride(0), _stream(stream)))


def fq_layernorm(x, gamma, beta, y, eps=1e-5, stream=None):
    M, h = x.shape
    _check(_lib.fq_layernorm(_ptr(x), M, h, x.stride(0), _ptr(gamma), _ptr(beta), eps, _ptr(y), y.stride(0),
                             _stream(stream)))


def fq_synth_normal_f16(dst, seed, stream_id, sigma, first=0, stream=None):
    _check(_lib.fq_synth_normal_f16(_ptr(dst), dst.numel(), seed, stream_id, first, sigma, _stream(stream)))


def fq_synth_token_ids(dst, seed, stream_id, vocab, stream=None):
    _check(_lib.fq_synth_token_ids(_ptr(dst), dst.numel(), seed, stream_id, vocab, _stream(stream)))


FQ_KC_ALL = 0xFF


def fq_timing_start(classes=None):
    """Record the launches of the named kernel classes (None: every class)."""
    mask = FQ_KC_ALL if classes is None else sum(1 << KERNEL_CLASSES.index(c) for c in classes)
    _check(_lib.fq_timing_start(mask))


def fq_timing_stop():
    """Returns {class name: dict(launches, seconds, flops, bytes, dropped)}."""
    arr = (fq_kernel_stats * len(KERNEL_CLASSES))()
    _check(_lib.fq_timing_stop(arr))
    return {n: {"launches": arr[i].launches, "seconds": arr[i].seconds, "flops": arr[i].flops,
                "bytes": arr[i].bytes, "dropped": arr[i].dropped} for i, n in enumerate(KERNEL_CLASSES)}


class Model:
    """Owner of an fq_model handle (fq_model_create / fq_model_destroy)."""

    def __init__(self, hidden, heads, ffn, layers, vocab=0, max_pos=0, compress_weight=True, resident_layers=-1,
                 host_layers=0, overlap=True, max_tokens=16384, compress_cache=True, cache_resident_layers=-1):
        self.cfg = fq_model_config(hidden, heads, ffn, layers, vocab, max_pos)
        self.pol = fq_policy(int(compress_weight), int(compress_cache), resident_layers, host_layers, int(overlap),
                             max_tokens, cache_resident_layers)
        h = c_vp()
        _check(_lib.fq_model_create(ctypes.byref(self.cfg), ctypes.byref(self.pol), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _lib.fq_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def init_random(self, seed, bias_sigma=0.0, stream=None):
        _check(_lib.fq_model_init_random(self.handle, seed, bias_sigma, _stream(stream)))

    def set_layer(self, layer, params, stream=None):
        """params: dict of device fp16 tensors with the fq_layer_weights field names."""
        w = fq_layer_weights(*[c_vp(params[n].data_ptr()) for n, _ in fq_layer_weights._fields_])
        _check(_lib.fq_model_set_layer(self.handle, layer, ctypes.byref(w), _stream(stream)))

    def set_embeddings(self, embed, pos, lnf_g, lnf_b, stream=None):
        _check(_lib.fq_model_set_embeddings(self.handle, _ptr(embed), _ptr(pos), _ptr(lnf_g), _ptr(lnf_b),
                                            _stream(stream)))

    def set_capture(self, captures):
        """captures: list of dict(layer, b0, nb, capacity, x_in, y_out, k16, v16, x1) with device fp16
        tensors [nb, capacity, hidden] (or None) -- see fq_model_set_capture.  [] clears."""
        arr = (fq_capture * max(1, len(captures)))()
        keep = []
        for i, c in enumerate(captures):
            arr[i] = fq_capture(c["layer"], c["b0"], c["nb"], c["capacity"],
                                *[_ptr(c.get(n)) for n in ("x_in", "y_out", "k16", "v16", "x1")])
            keep += [c.get(n) for n in ("x_in", "y_out", "k16", "v16", "x1")]
        _check(_lib.fq_model_set_capture(self.handle, arr if captures else None, len(captures)))
        self._capture_keep = keep

    def packed_weight(self, layer, which):
        p = fq_packed()
        _check(_lib.fq_model_packed_weight(self.handle, layer, which, ctypes.byref(p)))
        return p


class KVCache:
    """Owner of an fq_kv handle for every layer of a model."""

    def __init__(self, model, batch, capacity):
        h = c_vp()
        _check(_lib.fq_kv_create(model.handle, batch, capacity, ctypes.byref(h)))
        self.handle = h
        self.layers = model.cfg.layers

    def view(self, layer):
        v = fq_kv_layer()
        _check(_lib.fq_kv_layer_view(self.handle, layer, ctypes.byref(v)))
        return v

    def close(self):
        if self.handle:
            _lib.fq_kv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fq_layer_step(model, layer, kv, b0, B, T, pos, x, y, stream=None):
    _check(_lib.fq_layer_step(model.handle, layer, kv.handle, b0, B, T, pos, _ptr(x), _ptr(y), _stream(stream)))


_PROGRESS_FN = ctypes.CFUNCTYPE(None, c_i64, c_i64, c_vp)
_progress_keep = None


def fq_set_progress(fn):
    """fn(done, total) is called as each generated token's step finishes on
    the device during fq_generate; None disables it."""
    global _progress_keep
    if fn is None:
        _progress_keep = None
        _lib.fq_set_progress(None, None)
        return
    _progress_keep = _PROGRESS_FN(lambda done, total, user: fn(done, total))
    _lib.fq_set_progress(ctypes.cast(_progress_keep, c_vp), None)


def fq_generate(model, kv, prompt_ids, gen_len, logits=None, stream=None):
    """prompt_ids: host int32 tensor/ndarray [B, P].  Returns (out_ids int32 [B, gen_len], fq_gen_stats)."""
    import numpy as np
    ids = np.ascontiguousarray(np.asarray(prompt_ids, dtype=np.int32))
    B, P = ids.shape
    out = np.zeros((B, gen_len), np.int32)
    st = fq_gen_stats()
    _check(_lib.fq_generate(model.handle, kv.handle, ids.ctypes.data_as(_P(c_i32)), B, P, gen_len,
                            out.ctypes.data_as(_P(c_i32)), _ptr(logits), ctypes.byref(st), _stream(stream)))
    return out, st
