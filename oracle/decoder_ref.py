"""CPU oracle of the decoder layer around the rotated sparse linears.

TEST INFRASTRUCTURE ONLY (same rules as larosa_ref: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; it shares no code
with the HIP path).

The pages describe no transformer internals: they apply the rotated Top-K
sparsification to every linear layer's input of a pretrained decoder (LaRoSA
summary page, 方法详解 · 技术框架). The layer around those linears follows the
LLaMA-style decoder the workloads name, with these readings:
  * RMSNorm with unit gain and eps = 1e-5;
  * rotary position embedding on q and k, base 10000, "rotate-half" pairing
    (channel i with channel i + d_head/2 inside each head), the new token at
    position = number of cached positions;
  * single-query softmax attention of each head over its cached keys/values
    plus the new token's own key/value, scores scaled by 1/sqrt(d_head); a
    query head h reads key/value head h // (n_heads / n_kv_heads);
  * each step's output rounded to the activation dtype (bf16), fp64 inside.
Layouts: activations [B, D]; the key/value cache [B, n_kv_heads, T, d_head].
"""
from __future__ import annotations

import numpy as np

from . import larosa_ref as ref


def rmsnorm(h, eps: float = 1e-5, out_dtype: str = "bf16") -> np.ndarray:
    """h / sqrt(mean(h²) + eps), per token."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return ref.round_to(h / np.sqrt(ms + eps), out_dtype)


def rope_exact(x, n_heads: int, d_head: int, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotate-half rotary embedding of x [B, n_heads·d_head] at position pos
    (a scalar or one position per token), in float64 with no rounding."""
    x = np.asarray(x, dtype=np.float64)
    B = x.shape[0]
    half = d_head // 2
    xh = x.reshape(B, n_heads, d_head)
    freq = theta ** (-2.0 * np.arange(half) / d_head)            # ω_i
    p = np.broadcast_to(np.asarray(pos, dtype=np.float64), (B,))
    ang = p[:, None] * freq[None, :]                             # [B, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = xh[..., :half], xh[..., half:]
    out = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return out.reshape(B, n_heads * d_head)


def rope(x, n_heads, d_head, pos, theta=10000.0, out_dtype="bf16") -> np.ndarray:
    return ref.round_to(rope_exact(x, n_heads, d_head, pos, theta), out_dtype)


def decode_attention(q, k_new, v_new, k_cache, v_cache, n_heads: int, n_kv_heads: int,
                     d_head: int, out_dtype: str = "bf16") -> np.ndarray:
    """q [B, H·dh]; k_new, v_new [B, Hkv·dh]; caches [B, Hkv, T, dh].
    Returns [B, H·dh]."""
    q = np.asarray(q, dtype=np.float64)
    B = q.shape[0]
    qh = q.reshape(B, n_heads, d_head)
    kn = np.asarray(k_new, dtype=np.float64).reshape(B, n_kv_heads, 1, d_head)
    vn = np.asarray(v_new, dtype=np.float64).reshape(B, n_kv_heads, 1, d_head)
    K = np.concatenate([np.asarray(k_cache, dtype=np.float64), kn], axis=2)  # [B, Hkv, T+1, dh]
    Vv = np.concatenate([np.asarray(v_cache, dtype=np.float64), vn], axis=2)
    group = n_heads // n_kv_heads
    out = np.empty((B, n_heads, d_head))
    for h in range(n_heads):
        g = h // group
        s = np.einsum("bd,btd->bt", qh[:, h], K[:, g]) / np.sqrt(d_head)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h] = np.einsum("bt,btd->bd", p, Vv[:, g])
    return ref.round_to(out.reshape(B, n_heads * d_head), out_dtype)


def residual_add(h, o, out_dtype: str = "bf16") -> np.ndarray:
    return ref.round_to(np.asarray(h, dtype=np.float64) + np.asarray(o, dtype=np.float64),
                        out_dtype)
