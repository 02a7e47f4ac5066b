"""NumPy implementation of the counter-based input generator (see package docstring)."""
import math

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15          # SplitMix64 increment (odd, ~2**64 / golden ratio)
_M1 = 0xBF58476D1CE4E5B9            # SplitMix64 finaliser multipliers
_M2 = 0x94D049BB133111EB
LANE_SUM_STD = math.sqrt((65536.0 * 65536.0 - 1.0) / 3.0)

# Stream identifiers: one stream per tensor, so any element of any tensor can
# be regenerated from (seed, stream, flat index) alone.
TENSOR = {
    "w_qkv": 0, "w_out": 1, "w_fc1": 2, "w_fc2": 3,
    "b_qkv": 4, "b_out": 5, "b_fc1": 6, "b_fc2": 7,
    "ln1_g": 8, "ln1_b": 9, "ln2_g": 10, "ln2_b": 11,
}
STREAM = {
    "hidden": 1 << 20,        # C1/C2 hidden-state stream [B, P+T, h]
    "prompt": (1 << 20) + 1,  # token ids [B, P]
    "embed": (1 << 20) + 2,   # token embedding [V, h]
    "pos": (1 << 20) + 3,     # learned positions [P+G+2, h]
    "lnf_g": (1 << 20) + 4,
    "lnf_b": (1 << 20) + 5,
    "aux": (1 << 20) + 16,    # free streams for tests: aux + k
}


def layer_stream(layer: int, tensor: str) -> int:
    """Stream id of one per-layer tensor."""
    return layer * 64 + TENSOR[tensor]


def mix64(z):
    """SplitMix64 output function on a uint64 ndarray (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    """Key of one stream: mix64(seed * GAMMA + stream)."""
    return _mix64_int((seed * GAMMA + stream) & MASK64)


def raw_u64(seed: int, stream: int, index) -> np.ndarray:
    """64-bit outputs at the given flat indices (any integer array)."""
    idx = np.asarray(index, dtype=np.uint64)
    key = np.uint64(stream_key(seed, stream))
    with np.errstate(over="ignore"):
        ctr = key + (idx + np.uint64(1)) * np.uint64(GAMMA)
    return mix64(ctr)


def normal_scale_f32(sigma: float) -> np.float32:
    """fp32 multiplier that maps the centred lane sum to standard deviation sigma."""
    return np.float32(sigma / LANE_SUM_STD)


def normal_f16(seed: int, stream: int, shape=None, sigma: float = 1.0, index=None,
               chunk: int = 1 << 24, workers: int = 1) -> np.ndarray:
    """fp16 variates with std ``sigma``: either a whole tensor of ``shape`` (flat
    indices 0..n-1, row-major) or the elements at flat ``index``.  A whole tensor
    is produced in chunks of flat indices, on ``workers`` threads if more than one
    (every element depends only on its own index, so the result is the same)."""
    if index is None:
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float16)

        def part(s):
            e = min(n, s + chunk)
            out[s:e] = normal_f16(seed, stream, sigma=sigma, index=np.arange(s, e, dtype=np.uint64))
        if workers > 1:
            chunk = min(chunk, 1 << 22)  # enough pieces to keep every thread busy
        starts = range(0, n, chunk)
        if workers > 1 and n > chunk:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(part, starts))
        else:
            for s in starts:
                part(s)
        return out.reshape(shape)
    u = raw_u64(seed, stream, index)
    m = np.uint64(0xFFFF)
    lane_sum = ((u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m)
                + (u >> np.uint64(48))).astype(np.int64) - 131070
    return (lane_sum.astype(np.float32) * normal_scale_f32(sigma)).astype(np.float16)


def token_ids(seed: int, stream: int, shape, vocab: int) -> np.ndarray:
    """Uniform token ids in [0, vocab) as int32, flat indices 0..n-1."""
    n = int(np.prod(shape))
    u = raw_u64(seed, stream, np.arange(n, dtype=np.uint64))
    with np.errstate(over="ignore"):
        ids = ((u >> np.uint64(32)) * np.uint64(vocab)) >> np.uint64(32)
    return ids.astype(np.int32).reshape(shape)


def _unit_open(u):
    """Uniform variates in (0, 1) from 64-bit outputs: the top 53 bits plus half a step."""
    return ((u >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def heavy_tailed_f16(seed: int, stream: int, shape, sigma: float, kind: str) -> np.ndarray:
    """Heavy-tailed fp16 variates of scale ``sigma`` (test inputs whose
    quantisation groups span a wide range, unlike the bounded normal_f16):
      "student_t3": Student's t with 3 degrees of freedom, Z / sqrt(chi2_3 / 3);
      "laplace":    Laplace with scale sigma / sqrt(2) (std sigma), by inversion;
      "outliers":   normal variates (Box-Muller) with every 64th one, at a
                    pseudo-random place, multiplied by 40.
    Four uniforms per element come from flat counters 4i .. 4i+3 of the stream;
    the result is computed in float64 and rounded once to fp16."""
    n = int(np.prod(shape))
    ctr = np.arange(4 * n, dtype=np.uint64)
    u = _unit_open(raw_u64(seed, stream, ctr)).reshape(n, 4)

    def box_muller(a, b):
        r = np.sqrt(-2.0 * np.log(a))
        return r * np.cos(2.0 * np.pi * b), r * np.sin(2.0 * np.pi * b)

    if kind == "student_t3":
        z0, z1 = box_muller(u[:, 0], u[:, 1])
        z2, z3 = box_muller(u[:, 2], u[:, 3])
        x = z0 / np.sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0) * sigma
    elif kind == "laplace":
        c = u[:, 0] - 0.5
        x = -np.sign(c) * np.log1p(-2.0 * np.abs(c)) * (sigma / math.sqrt(2.0))
    elif kind == "outliers":
        z0, _ = box_muller(u[:, 0], u[:, 1])
        x = z0 * sigma * np.where(u[:, 2] < 1.0 / 64.0, 40.0, 1.0)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    return np.clip(x, -65504.0, 65504.0).astype(np.float16).reshape(shape)
