"""Oracle: tree-masked attention (fp64, C loops).  Test infrastructure only.

Wiblog "Medusa multi-head speculative decoding", tree-attention section, and Ultralytics
"Medusa Heads", tree-attention section: all candidate tokens are verified in one forward pass;
each token attends to the prefix and to its own ancestors in the tree only.

Readings where the pages are silent: scale 1/sqrt(D) by default, no bias; the tree tokens' K/V
sit at cache rows prefix_len[b] .. prefix_len[b]+T-1 in node order; grouped heads map query
head hq to kv head hq // (Hq // Hkv).
"""

import numpy as np

from . import _clib


def tree_attention(q, k_cache, v_cache, dtype, prefix_len, mask, Hkv, scale=None, sel=None):
    """q [B,Hq,T,D]; caches [B,Hkv,Lcap,D]; mask [T][W] (list of ints or uint64 array).

    Returns out [B,Hq,T,D] fp64.  With sel (array of (b, hq, i) rows) only those units are
    computed; the others are NaN."""
    for a in (q, k_cache, v_cache):
        _clib.check_input(a, dtype)
    B, Hq, T, D = q.shape
    assert D <= 256 and Hq % Hkv == 0
    lcap = k_cache.shape[2]
    assert k_cache.shape == (B, Hkv, lcap, D) and v_cache.shape == k_cache.shape
    m = np.ascontiguousarray(np.array(mask, dtype=np.uint64))
    assert m.shape[0] == T
    W = m.shape[1]
    pl = np.ascontiguousarray(prefix_len, np.int32)
    assert pl.shape == (B,) and int(pl.max()) + T <= lcap
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.full((B, Hq, T, D), np.nan, np.float64)
    if sel is not None:
        sel = np.ascontiguousarray(sel, np.int32).reshape(-1, 3)
    _clib.lib().oracle_tree_attention(
        _clib.vptr(q), _clib.vptr(k_cache), _clib.vptr(v_cache), _clib.DT[dtype], _clib.vptr(pl),
        B, Hq, Hkv, T, D, lcap, _clib.vptr(m), W, scale, _clib.vptr(sel),
        0 if sel is None else sel.shape[0], _clib.dptr(out))
    return out
