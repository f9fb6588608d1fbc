"""Oracle: Medusa heads and per-head top-k (fp64).  Test infrastructure only.

Ultralytics glossary "Medusa Heads", section on how the heads predict the next tokens: every
head reads the same last hidden state h, applies one fully connected layer with SiLU and a
residual connection, then a vocab projection; the code sample there uses Linear(hidden, hidden)
with a bias for W1 and Linear(hidden, vocab) without a bias for W2 ([out, in] weights), so
  logits_k = W2_k (h + SiLU(W1_k h + b1_k)).
Wiblog "Medusa multi-head speculative decoding", inference-flow section: each head outputs its
top-k candidate tokens.  The pages do not order equal logits; here ties go to the lower id.
"""

import numpy as np

from . import _clib


def project(w, dtype, x):
    """out[b, v] = sum_j w[v, j] x[b, j] in fp64.  w [rows, hd] (stored dtype), x [B, hd] f64."""
    _clib.check_input(w, dtype)
    x = np.ascontiguousarray(x, np.float64)
    B, hd = x.shape
    rows = w.shape[0]
    assert w.shape == (rows, hd)
    out = np.empty((B, rows), np.float64)
    _clib.lib().oracle_project(_clib.vptr(w), _clib.DT[dtype], rows, hd, _clib.dptr(x), hd, B,
                               _clib.dptr(out), rows)
    return out


def heads(h, w1, b1, w2, dtype):
    """Returns (r [B,K,Hd], logits [B,K,V]) in fp64 for inputs in their stored dtype."""
    for a in (h, w1, b1, w2):
        _clib.check_input(a, dtype)
    B, hd = h.shape
    K, V = w2.shape[0], w2.shape[1]
    assert w1.shape == (K, hd, hd) and b1.shape == (K, hd) and w2.shape == (K, V, hd)
    r = np.empty((B, K, hd), np.float64)
    logits = np.empty((B, K, V), np.float64)
    _clib.lib().oracle_heads(_clib.vptr(h), _clib.vptr(w1), _clib.vptr(b1), _clib.vptr(w2),
                             _clib.DT[dtype], B, hd, V, K, _clib.dptr(r), _clib.dptr(logits))
    return r, logits


def topk(x, k):
    """Top-k over the last axis: ids sorted by value descending, equal values -> lower id."""
    x = np.ascontiguousarray(x, np.float64)
    lead = x.shape[:-1]
    n = x.shape[-1]
    assert 1 <= k <= n
    rows = int(np.prod(lead)) if lead else 1
    ids = np.empty(lead + (k,), np.int32)
    vals = np.empty(lead + (k,), np.float64)
    _clib.lib().oracle_topk(_clib.dptr(x), rows, n, k, _clib.vptr(ids), _clib.dptr(vals))
    return ids, vals


def topk_ties(logits64, k, rel=1e-4):
    """Per row, True where two adjacent values among the oracle's ranks 0..k (k-1 vs k included)
    are within rel*max(1,|v|): the top-k id set or order is then not fixed by fp64 vs fp32."""
    n = logits64.shape[-1]
    kk = min(k + 1, n)
    _, vals = topk(logits64, kk)
    gap = vals[..., :-1] - vals[..., 1:]
    tol = rel * np.maximum(1.0, np.abs(vals[..., :-1]))
    return np.any(gap <= tol, axis=-1)
