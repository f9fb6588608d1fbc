"""Oracle: Medusa heads made of several residual blocks, optionally with LayerNorm (fp64).
Test infrastructure only.

Wiblog "Medusa multi-head speculative decoding", heads section: a head is usually one or more
residual blocks followed by a linear layer, a block being LayerNorm and a feed-forward network.
Ultralytics "Medusa Heads", how-the-heads-predict section: the block is one fully connected
layer (with bias) with SiLU and a residual connection, then the vocab projection (no bias).

Readings where the pages stop:
  * block j of head k:  x <- x + SiLU(W1[k][j] n(x) + b1[k][j]), starting from x = h;
    n(x) = x without LayerNorm, else n(x) = (x - mean) / sqrt(var + eps) * gamma + beta over the
    hidden dimension, var the mean squared deviation (torch's LayerNorm), eps 1e-5;
  * the vocab projection reads the last block's x; no norm after the last block;
  * weights [K][n_blocks][out][in] with n_blocks = 1 and no LayerNorm being the single-block
    heads of the rest of the step.
"""

import numpy as np

from . import bf16
from .heads import project

_f64 = bf16.to_f64


def layer_norm(x, gamma, beta, eps):
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def heads_blocks(h, w1, b1, w2, dtype, gamma=None, beta=None, eps=1e-5):
    """h [B,Hd]; w1 [K,nb,Hd,Hd]; b1 [K,nb,Hd]; w2 [K,V,Hd]; gamma, beta [K,nb,Hd] or None
    (inputs in their stored dtype; h may also be fp64).  Returns (r [B,K,Hd] after the last
    block, logits [B,K,V]) in fp64."""
    K, nb, hd, _ = w1.shape
    assert b1.shape == (K, nb, hd) and w2.shape[0] == K and w2.shape[2] == hd
    assert (gamma is None) == (beta is None)
    h64 = _f64(h, dtype)
    B = h64.shape[0]
    V = w2.shape[1]
    r = np.empty((B, K, hd))
    logits = np.empty((B, K, V))
    for k in range(K):
        x = h64.copy()
        for j in range(nb):
            inp = x if gamma is None else layer_norm(x, _f64(gamma[k, j], dtype),
                                                     _f64(beta[k, j], dtype), eps)
            u = project(np.ascontiguousarray(w1[k, j]), dtype, inp) + _f64(b1[k, j], dtype)
            x = x + u / (1.0 + np.exp(-u))
        r[:, k] = x
        logits[:, k] = project(np.ascontiguousarray(w2[k]), dtype, x)
    return r, logits
