"""Oracle: rotary position embedding of the tree tokens at their depth positions (fp64, numpy).
Test infrastructure only.

Wiblog "Medusa multi-head speculative decoding", tree-attention section: besides the mask, the
position encoding has to follow the tree so that every token gets its correct position index,
i.e. the position it would have in plain sequential decoding of its own path: prefix_len + depth.

Readings where the pages are silent (they never name the encoding):
  * the encoding is the rotary one of the LLaMA-family models the workloads are shaped after:
    dimension i < D/2 is paired with i + D/2 and the pair (x_i, x_{i+D/2}) is turned by the
    angle pos * base^(-2i/D), base 10000 unless given;
  * the prefix keys in the cache were rotated when they were written; the tree tokens' query
    rows and their key rows in the cache (prefix_len .. prefix_len + T - 1) are rotated here,
    the keys in place, and both are rounded to the step dtype (nearest even for bf16) before
    attention uses them.
"""

import numpy as np

from . import bf16
from .attention import tree_attention


def rope(x, pos, base=10000.0):
    """x [..., D] (fp64 or anything castable), pos broadcastable to x.shape[:-1]; fp64 result."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.asarray(pos, np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _round(x, dtype):
    return bf16.round_rne(x) if dtype == "bf16" else x.astype(np.float32)


def _decode(x, dtype):
    return bf16.to_f64(x, dtype)


def rotate_tree(q, k_cache, dtype, prefix_len, position_ids, base=10000.0):
    """Returns (q_rot, k_cache_rot) in the storage dtype: q [B,Hq,T,D] rotated at
    position_ids [B,T]; the cache's tree rows rotated likewise; other rows unchanged."""
    B, Hq, T, D = q.shape
    pos = np.asarray(position_ids, np.int64)
    qr = _round(rope(_decode(q, dtype), pos[:, None, :], base), dtype)
    kr = k_cache.copy()
    for b in range(B):
        L = int(prefix_len[b])
        rows = _decode(k_cache[b, :, L:L + T], dtype)
        kr[b, :, L:L + T] = _round(rope(rows, pos[b][None, :], base), dtype)
    return qr, kr


def tree_attention_rope(q, k_cache, v_cache, dtype, prefix_len, mask, Hkv, position_ids,
                        base=10000.0, scale=None):
    """Rotates the tree tokens' queries and keys, then tree attention.  Returns
    (out [B,Hq,T,D] fp64, k_cache with the rotated tree rows)."""
    qr, kr = rotate_tree(q, k_cache, dtype, prefix_len, position_ids, base)
    return tree_attention(qr, kr, v_cache, dtype, prefix_len, mask, Hkv, scale=scale), kr
