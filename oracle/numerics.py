"""Textbook numerics in fp64 with the contract's rounding points.

Arrays hold float64 values; "rounding to fp32" keeps them float64 but
representable in fp32. All functions here are the plain definitions.
"""
from __future__ import annotations

import numpy as np


def to_f32(x):
    """Round to the nearest fp32 value (IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_bf16(x):
    """Round to fp32, then to bf16 by round-to-nearest-even on the bit pattern."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def operand(x, dtype: str):
    """An activation entering a matrix product: fp32 for both dtypes (only
    the weights are stored in bf16)."""
    return to_f32(x)


def kv_store(x, dtype: str):
    """K and V as written to the cache: fp32 for both dtypes."""
    return to_f32(x)


def rmsnorm(h, gain, eps: float):
    """x / sqrt(mean(x^2) + eps) * gain, over the last axis."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * gain


def silu(x):
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def rope_tables(positions, head_dim: int, base: float):
    """cos/sin of p * base^(-2i/d), i < d/2, computed in fp64, rounded to fp32."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    return to_f32(np.cos(ang)), to_f32(np.sin(ang))


def apply_rope(x, cos, sin):
    """Rotate-half RoPE. x [M, heads, d]; cos/sin [M, d/2]."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def log_softmax(logits):
    """l - max - log(sum(exp(l - max))) over the last axis, in fp64."""
    z = np.asarray(logits, dtype=np.float64)
    mx = np.max(z, axis=-1, keepdims=True)
    return z - mx - np.log(np.sum(np.exp(z - mx), axis=-1, keepdims=True))
