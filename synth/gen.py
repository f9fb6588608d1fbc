"""Seeded generators.  Every draw comes from numpy's PCG64 in independent 2**22-element blocks.

Recipe:
  * A tensor is filled block by block (2**22 elements, row-major order).  Block i of tensor t of
    stream s draws float32 standard normals from Generator(PCG64(SeedSequence([seed, s, t, i]))),
    so blocks can be drawn in parallel threads and any block can be regenerated alone.
  * Normals are scaled by their std in fp32, then rounded to bf16 with round-to-nearest-even when
    the workload is bf16.  bf16 tensors are held as uint16 bit patterns.
  * stream 0: h [B,Hd] ~ N(0,1)                                       (tensor 0)
  * stream 1: head k: W1[k] [Hd,Hd] (tensor 3k), b1[k] [Hd] (3k+1), W2[k] [V,Hd] (3k+2),
              all ~ N(0, w_std^2)
  * stream 2: K cache (tensor 0), V cache (tensor 1) [B,Hkv,Lcap,D] ~ N(0,1); rows [0, L_b) are
              the prefix, rows past L_b+T are filler that a correct kernel never reads
  * stream 3: tree Q [B,Hq,T,D] (tensor 0), tree K (1), tree V (2) [B,Hkv,T,D] ~ N(0,1); tree
              K/V are written over cache rows [L_b, L_b+T)
  * stream 4: root tokens [B], uniform integers in [0,V)
  * stream 5: verification logits [B,T,V] ~ N(0, logit_std^2)        (tensor 0)
  * stream 6: one uniform per (b, non-root node) in node order; the node's own token gets
              +boost in its parent's row when the draw is below boost_p.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def rng_for(seed, stream, tensor=0, block=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), int(stream), int(tensor), int(block)])))


def f32_to_bf16_bits(a):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_block(out_flat, seed, stream, tensor, i, std, dtype):
    s = i * BLOCK
    m = min(BLOCK, out_flat.size - s)
    x = rng_for(seed, stream, tensor, i).standard_normal(m, dtype=np.float32)
    x *= np.float32(std)
    out_flat[s:s + m] = f32_to_bf16_bits(x) if dtype == "bf16" else x


def fill_normals(out, seed, stream, tensor, std, dtype):
    flat = out.reshape(-1)
    nb = (flat.size + BLOCK - 1) // BLOCK
    if nb <= 1:
        for i in range(nb):
            _fill_block(flat, seed, stream, tensor, i, std, dtype)
    else:
        with ThreadPoolExecutor(min(_THREADS, nb)) as ex:
            list(ex.map(lambda i: _fill_block(flat, seed, stream, tensor, i, std, dtype), range(nb)))
    return out


def _empty(shape, dtype):
    return np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)


def normals(shape, seed, stream, tensor, std, dtype):
    return fill_normals(_empty(shape, dtype), seed, stream, tensor, std, dtype)


def gen_head_inputs(cfg, seed=None):
    """h [B,Hd]; W1 [K,Hd,Hd] ([out,in]); b1 [K,Hd]; W2 [K,V,Hd] ([out,in])."""
    seed = cfg.seed if seed is None else seed
    h = normals((cfg.B, cfg.Hd), seed, 0, 0, 1.0, cfg.dtype)
    w1 = _empty((cfg.K, cfg.Hd, cfg.Hd), cfg.dtype)
    b1 = _empty((cfg.K, cfg.Hd), cfg.dtype)
    w2 = _empty((cfg.K, cfg.V, cfg.Hd), cfg.dtype)
    for k in range(cfg.K):
        fill_normals(w1[k], seed, 1, 3 * k, cfg.w_std, cfg.dtype)
        fill_normals(b1[k], seed, 1, 3 * k + 1, cfg.w_std, cfg.dtype)
        fill_normals(w2[k], seed, 1, 3 * k + 2, cfg.w_std, cfg.dtype)
    return dict(h=h, w1=w1, b1=b1, w2=w2)


def gen_root_tokens(cfg, seed=None):
    seed = cfg.seed if seed is None else seed
    return rng_for(seed, 4).integers(0, cfg.V, size=cfg.B).astype(np.int32)


def gen_attention_inputs(cfg, T, seed=None, prefix_lens=None, lcap=None):
    """Q [B,Hq,T,D]; K/V cache [B,Hkv,Lcap,D] holding the prefix at rows [0,L_b) and the tree
    tokens' K/V at rows [L_b, L_b+T) in node order; rows past that are filler."""
    seed = cfg.seed if seed is None else seed
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    pl = np.full(B, cfg.L, np.int32) if prefix_lens is None else np.asarray(prefix_lens, np.int32)
    assert pl.shape == (B,)
    need = int(pl.max()) + T
    lcap = need if lcap is None else int(lcap)
    assert lcap >= need
    kc = normals((B, Hkv, lcap, D), seed, 2, 0, 1.0, cfg.dtype)
    vc = normals((B, Hkv, lcap, D), seed, 2, 1, 1.0, cfg.dtype)
    q = normals((B, Hq, T, D), seed, 3, 0, 1.0, cfg.dtype)
    kt = normals((B, Hkv, T, D), seed, 3, 1, 1.0, cfg.dtype)
    vt = normals((B, Hkv, T, D), seed, 3, 2, 1.0, cfg.dtype)
    for b in range(B):
        kc[b, :, pl[b]:pl[b] + T] = kt[b]
        vc[b, :, pl[b]:pl[b] + T] = vt[b]
    return dict(q=q, k_cache=kc, v_cache=vc, prefix_len=pl, lcap=lcap)


def gen_verif_logits(cfg, parent, tokens, seed=None):
    """Verification logits [B,T,V]: row n is the model's distribution after tree node n.

    parent [T] (parent[0] = -1) and tokens [B,T] describe the tree of this step; they are
    inputs here (whichever side computed them), not derived.  A node c's own token gets
    +boost in row parent[c] with probability boost_p."""
    seed = cfg.seed if seed is None else seed
    parent = np.asarray(parent)
    tokens = np.asarray(tokens)
    B, V = cfg.B, cfg.V
    T = parent.shape[0]
    x = normals((B, T, V), seed, 5, 0, cfg.logit_std, "f32")
    u = rng_for(seed, 6).random((B, T - 1))
    for b in range(B):
        for c in range(1, T):
            if u[b, c - 1] < cfg.boost_p:
                x[b, parent[c], tokens[b, c]] += np.float32(cfg.boost)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(x).reshape(B, T, V)
    return x
