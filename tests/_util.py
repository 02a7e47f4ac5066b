"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

# Layer-output tolerance: relative L2 <= 5e-3 and max |err| <= 3e-2 against
# the oracle's float64 values (fp32 accumulation on the GPU).
REL_L2 = 5e-3
MAX_ABS = 3e-2


def dev(a):
    """numpy -> torch on cuda:0 (fp16 stays fp16, uint8 stays uint8)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.detach().cpu().numpy()


def empty_packed(rows, cols):
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((rows, cols // 64, 2), dtype=torch.float16, device="cuda:0")
    return codes, meta


def bits16(a):
    return np.asarray(a).view(np.uint16)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, rel=REL_L2, abs_=MAX_ABS, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(got, ref)
    m = float(np.abs(got - ref).max()) if got.size else 0.0
    assert r <= rel and m <= abs_, f"{what}: rel_l2={r:.3e} (<= {rel}), max_abs={m:.3e} (<= {abs_})"
    return r, m


def log(msg):
    print(msg, flush=True)


def ulp16(x):
    """Spacing of fp16 values at |x| (2^-24 in the subnormal range)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - 10)


def assert_layer_close(got, ref, resid=None, what=""):
    """An fp16 storage point of a layer against the oracle's float64 value
    before rounding: relative L2 <= 5e-3, and max |err| <= 3e-2 while the value
    (and the residual it adds, for y = x1 + FFN(x1)) stay below 16 in
    magnitude.  Above that the fp16 format itself moves the bound: the value
    carries its own rounding (half an ulp), and a residual that both sides
    round to fp16 may land one ulp apart (fp32 accumulation can move it
    across a rounding boundary); the bound grows by exactly the growth of
    those two terms beyond their size below 16 (half an ulp plus one ulp at
    2^-7).  Ulps are taken at the larger magnitude of the two sides (the GPU
    rounds at its own value's magnitude).  resid: the residual's magnitude per
    element (None for a value with no residual)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(got, ref)
    err = np.abs(got - ref)
    ymag = np.maximum(np.abs(got), np.abs(ref))
    storage = 0.5 * ulp16(ymag) + (0.0 if resid is None else ulp16(resid))
    storage16 = 0.5 * 2.0 ** -7 + (0.0 if resid is None else 2.0 ** -7)
    bound = MAX_ABS + np.maximum(0.0, storage - storage16)
    ratio = err / bound
    worst = float(ratio.max()) if err.size else 0.0
    at = np.unravel_index(int(ratio.argmax()), ratio.shape) if err.size else None
    detail = "" if at is None else (f" at {tuple(int(i) for i in at)}: gpu {got[at]:.6g} oracle {ref[at]:.6g}" +
                                    ("" if resid is None else f" |x1| {np.asarray(resid)[at]:.6g}") +
                                    f" bound {bound[at]:.4g}")
    assert r <= REL_L2 and worst <= 1.0, \
        f"{what}: rel_l2={r:.3e} (<= {REL_L2}), max |err|/bound={worst:.3f} (max |err| {err.max():.3e}){detail}"
    return r, float(err.max()) if err.size else 0.0, float(np.abs(ref).max()) if ref.size else 0.0, detail


def copy_dev(dst, src, nbytes):
    """hipMemcpy with hipMemcpyDefault between raw addresses (device or pinned host)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), ctypes.c_size_t(nbytes), 4) == 0


def gpu_cache(view, nb, cap):
    """Sequences 0..nb-1 of one cache layer (an fq_kv_layer view), copied to the host:
    4-bit codes and {min, scale} (as fp16) or the fp16 entries, keyed like the
    oracle's cache.  The view's capacity must be cap."""
    H, d = view.heads, view.head_dim
    assert view.capacity == cap
    if view.bits == 16:
        items = (("k", view.k16, (nb, H, cap, d), torch.float16), ("v", view.v16, (nb, H, cap, d), torch.float16))
    else:
        items = (("k_codes", view.k_codes, (nb, H, cap, d // 2), torch.uint8),
                 ("v_codes", view.v_codes, (nb, H, cap, d // 2), torch.uint8),
                 ("k_meta", view.k_meta, (nb, H, cap, d // 64, 2), torch.float16),
                 ("v_meta", view.v_meta, (nb, H, cap, d // 64, 2), torch.float16))
    out = {}
    for name, ptr, shape, dt in items:
        t = torch.empty(shape, dtype=dt, device="cuda:0")
        copy_dev(t.data_ptr(), ptr, t.numel() * t.element_size())
        out[name] = host(t)
    return out


def packed_to_host(p):
    """An fq_packed on the device -> (codes uint8 [rows, cols/2], meta fp16 [rows, cols/64, 2])."""
    n, k = p.rows, p.cols
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device="cuda:0")
    torch.cuda.synchronize()
    copy_dev(codes.data_ptr(), p.codes, n * k // 2)
    copy_dev(meta.data_ptr(), p.meta, n * (k // 64) * 4)
    return host(codes), host(meta)


def assert_same_cache(gpu, ref, what):
    """Both caches bit for bit (codes, {min, scale} as uint16, or fp16 entries)."""
    for name, r in ref.items():
        g = gpu[name]
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        gb, rb = (g.view(np.uint16), r.view(np.uint16)) if r.dtype == np.float16 else (g, r)
        bad = np.argwhere(gb != rb)
        assert len(bad) == 0, f"{what} {name}: {len(bad)} entries differ, first {bad[:3].tolist()}"
