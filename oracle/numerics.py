"""Elementwise and row-wise definitions used by the oracle's forward pass.

Test infrastructure only (see the package docstring).

The pages fix the model family only loosely (a decoder LM with a KV cache,
MoE layers with top-k routing); the plainest reading adopted here is the
LLaMA/Qwen family: RMSNorm with a gain, rotate-half rotary embedding, causal
softmax attention with grouped KV heads, SwiGLU FFN.  Each function is the
textbook definition written out in float64 (or the dtype of its input).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Storage formats: reading them and rounding to them
# ----------------------------------------------------------------------------


def bf16_bits_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bit patterns (uint16) -> values.  A bf16 number is the upper half
    of an IEEE binary32, so the value is exact in any wider float."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits, ties to even),
    returned in x's float dtype.  Written from the definition: scale the
    significand to [128, 256), round half-to-even, scale back.  Values are
    far from bf16's overflow and subnormal range in this model."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return r


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x).astype(np.float32).astype(np.float64)


def round_kv(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Keys and values are stored in the cache in the model's KV dtype; the
    attention reads the stored (rounded) values for every position,
    including the current block."""
    if kv_dtype == "bf16":
        return round_to_bf16(x).astype(x.dtype)
    if kv_dtype == "f32":
        return np.asarray(x).astype(np.float32).astype(x.dtype)
    raise ValueError(kv_dtype)


def dequant_int4(packed: np.ndarray, scales: np.ndarray, group: int, dtype=np.float64) -> np.ndarray:
    """Group-wise symmetric int4: packed uint8 [K/2, N] (even k in the low
    nibble, two's complement), fp16 scales [K/group, N].  w = q * s."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = lo - 16 * (lo >= 8)
    hi = hi - 16 * (hi >= 8)
    K = 2 * p.shape[0]
    q = np.empty((K, p.shape[1]), dtype=dtype)
    q[0::2] = lo
    q[1::2] = hi
    s = np.asarray(scales, dtype=np.float16).astype(dtype)
    return q * np.repeat(s, group, axis=0)


# ----------------------------------------------------------------------------
# Layers
# ----------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[p, i] = pos_p * theta^(-2i/D), i < D/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing: for i < D/2 the pair
    (x_i, x_{i+D/2}) of the row at position p is rotated by angle[p, i].
    x: [m, H, D]; positions: [m]."""
    D = x.shape[-1]
    h = D // 2
    ang = rope_angles(positions, D, theta)           # [m, D/2]
    c = np.cos(ang)[:, None, :].astype(x.dtype)
    s = np.sin(ang)[:, None, :].astype(x.dtype)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    zmax = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - zmax)
    return e / np.sum(e, axis=axis, keepdims=True)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, L: int) -> np.ndarray:
    """Verification-block attention.

    q: [m, Hq, D] queries for positions L..L+m-1.
    K, V: [Hkv, T, D] with T >= L+m: cached keys/values, the block's own
    entries at L..L+m-1.  Query j attends to positions t <= L+j only (the
    backwards-only rule); query head h reads KV head floor(h*Hkv/Hq).
    Returns o: [m, Hq, D].
    """
    m, Hq, D = q.shape
    Hkv = K.shape[0]
    T = L + m
    t = np.arange(T)
    j = np.arange(m)
    visible = t[None, :] <= (L + j)[:, None]          # [m, T]
    o = np.empty_like(q)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = (q[:, h, :] @ K[g, :T, :].T) / np.sqrt(D)
        s = np.where(visible, s, -np.inf)
        p = softmax(s, axis=-1)
        o[:, h, :] = p @ V[g, :T, :]
    return o
