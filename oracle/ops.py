"""Dense operations of the layer, evaluated on dequantised values in float64.

These are plain definitions (matrix product, layer normalisation, softmax
attention); compressed operands enter only through quant.dequant_*.  The
pages say only that weights and cache are stored in 4 bits
(FlexGen README, "Extreme Compression"); computing on the reconstructed
values is the plainest reading of the inference/research record's
"Mechanism" field (compression is there so that more state fits on the GPU).
"""
import numpy as np

LN_EPS = 1e-5


def gemm(x16: np.ndarray, w16: np.ndarray, bias16=None) -> np.ndarray:
    """Y = X @ W^T (+ b) in float64.  X fp16 [M, K]; W fp16 [N, K] (already dequantised);
    bias fp16 [N] or None.  Returns float64 [M, N] before any rounding."""
    y = np.asarray(x16, dtype=np.float64) @ np.asarray(w16, dtype=np.float64).T
    if bias16 is not None:
        y = y + np.asarray(bias16, dtype=np.float64)[None, :]
    return y


def layernorm(x16: np.ndarray, gamma16: np.ndarray, beta16: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """(x - mean) / sqrt(biased var + eps) * gamma + beta over the last axis, float64."""
    x = np.asarray(x16, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma16, np.float64) + np.asarray(beta16, np.float64)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = s.max(axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def attention_decode(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray) -> np.ndarray:
    """One query per (batch, head) against `len` cached keys.

    q [B, H, d] (already scaled by d^-1/2); k_hat, v_hat [B, H, len, d] (dequantised cache).
    s_j = q . k_j ; p = softmax(s) ; o = sum_j p_j v_j.  Returns float64 [B, H, d]."""
    q = np.asarray(q, np.float64)
    s = np.einsum("bhd,bhjd->bhj", q, np.asarray(k_hat, np.float64))
    p = softmax(s, axis=-1)
    return np.einsum("bhj,bhjd->bhd", p, np.asarray(v_hat, np.float64))


def attention_prefill_causal(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray) -> np.ndarray:
    """Causal attention of T queries over the same T positions (query i sees keys 0..i).

    q [B, H, T, d] (scaled); k_hat, v_hat [B, H, T, d].  Returns float64 [B, H, T, d].
    Evaluated one batch entry at a time to bound memory."""
    B, H, T, d = q.shape
    out = np.empty((B, H, T, d), dtype=np.float64)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    for b in range(B):
        s = np.asarray(q[b], np.float64) @ np.swapaxes(np.asarray(k_hat[b], np.float64), -1, -2)
        s[:, mask] = -np.inf
        out[b] = softmax(s, axis=-1) @ np.asarray(v_hat[b], np.float64)
    return out
