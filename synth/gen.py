"""Seeded generators.  Every draw comes from numpy's PCG64, one stream per tensor group.

Recipe (stated once here and in the design notes):
  * stream = Generator(PCG64(SeedSequence([seed, stream_id]))).
  * Normals are drawn in fp64 in chunks of 2**24 elements, scaled, cast to fp32, then rounded
    to bf16 with round-to-nearest-even when the workload is bf16.  bf16 tensors are held as
    uint16 bit patterns.
  * stream 0: h [B,Hd] ~ N(0,1)
  * stream 1: for each head k in order: W1[k] [Hd,Hd], b1[k] [Hd], W2[k] [V,Hd], all ~ N(0, w_std^2)
  * stream 2: prefix K then prefix V, each [B,Hkv,L_b,D] ~ N(0,1) (per sequence b in order)
  * stream 3: tree Q [B,Hq,T,D], tree K, tree V [B,Hkv,T,D] ~ N(0,1)
  * stream 4: root tokens [B], uniform integers in [0,V)
  * stream 5: verification logits [B,T,V] ~ N(0, logit_std^2)
  * stream 6: one uniform per (b, non-root node) in node order; the node's own token gets
    +boost in the row of its parent when the draw is below boost_p.
  * stream 7: cache rows beyond L_b+T (never read by a correct kernel) ~ N(0,1)
"""

import numpy as np

CHUNK = 1 << 24


def rng_for(seed, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def f32_to_bf16_bits(a):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normals_into(rng, out_flat, std, dtype):
    """Fill out_flat (float32 or uint16 view) with N(0, std^2) draws, chunk by chunk."""
    n = out_flat.size
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        x = (rng.standard_normal(m) * std).astype(np.float32)
        if dtype == "bf16":
            out_flat[s:s + m] = f32_to_bf16_bits(x)
        else:
            out_flat[s:s + m] = x


def _empty(shape, dtype):
    return np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)


def normals(rng, shape, std, dtype):
    a = _empty(shape, dtype)
    _normals_into(rng, a.reshape(-1), std, dtype)
    return a


def gen_head_inputs(cfg, seed=None):
    """h [B,Hd]; W1 [K,Hd,Hd] ([out,in]); b1 [K,Hd]; W2 [K,V,Hd] ([out,in])."""
    seed = cfg.seed if seed is None else seed
    h = normals(rng_for(seed, 0), (cfg.B, cfg.Hd), 1.0, cfg.dtype)
    r1 = rng_for(seed, 1)
    w1 = _empty((cfg.K, cfg.Hd, cfg.Hd), cfg.dtype)
    b1 = _empty((cfg.K, cfg.Hd), cfg.dtype)
    w2 = _empty((cfg.K, cfg.V, cfg.Hd), cfg.dtype)
    for k in range(cfg.K):
        _normals_into(r1, w1[k].reshape(-1), cfg.w_std, cfg.dtype)
        _normals_into(r1, b1[k].reshape(-1), cfg.w_std, cfg.dtype)
        _normals_into(r1, w2[k].reshape(-1), cfg.w_std, cfg.dtype)
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
    kc = _empty((B, Hkv, lcap, D), cfg.dtype)
    vc = _empty((B, Hkv, lcap, D), cfg.dtype)
    r2 = rng_for(seed, 2)
    for cache in (kc, vc):
        for b in range(B):
            for g in range(Hkv):
                _normals_into(r2, cache[b, g, :pl[b]].reshape(-1), 1.0, cfg.dtype)
    r3 = rng_for(seed, 3)
    q = normals(r3, (B, Hq, T, D), 1.0, cfg.dtype)
    kt = normals(r3, (B, Hkv, T, D), 1.0, cfg.dtype)
    vt = normals(r3, (B, Hkv, T, D), 1.0, cfg.dtype)
    r7 = rng_for(seed, 7)
    for b in range(B):
        kc[b, :, pl[b]:pl[b] + T] = kt[b]
        vc[b, :, pl[b]:pl[b] + T] = vt[b]
        rest = lcap - (pl[b] + T)
        if rest > 0:
            for cache in (kc, vc):
                for g in range(Hkv):
                    _normals_into(r7, cache[b, g, pl[b] + T:].reshape(-1), 1.0, cfg.dtype)
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
    x = np.empty((B, T, V), np.float32)
    _normals_into(rng_for(seed, 5), x.reshape(-1), cfg.logit_std, "f32")
    u = rng_for(seed, 6).random((B, T - 1))
    for b in range(B):
        for c in range(1, T):
            if u[b, c - 1] < cfg.boost_p:
                x[b, parent[c], tokens[b, c]] += np.float32(cfg.boost)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(x).reshape(B, T, V)
    return x
