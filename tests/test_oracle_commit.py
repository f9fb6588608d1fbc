"""Pins for the oracle's commit of the accepted candidate.

Wiblog "Medusa multi-head speculative decoding", inference-flow section: the accepted prefix is
output and decoding continues from the last accepted token.  The commit is pinned by what must
hold afterwards, checked independently of how it is computed:
  * plain causal attention of each accepted node's query over cache rows [0, L + depth] of the
    committed cache equals what tree attention gave that node before the commit (the cache now
    holds exactly the accepted sequence, in order);
  * the emitted tokens are the root and the accepted nodes, found here by walking parent
    pointers up from the last accepted node;
  * rows outside L+1 .. L+a are untouched; accept length 0 moves nothing.
"""

import numpy as np
import pytest

import oracle
from synth.configs import custom
from synth.gen import gen_attention_inputs, rng_for
from synth.trees import cartesian_choices, load_tree_choices


def _setup(tree, B, Hq, Hkv, D, pls, seed, topk=10, K=5):
    st = oracle.build_static(load_tree_choices(tree) if isinstance(tree, str) else tree, topk, K)
    T = st["T"]
    cfg = custom(B=B, Hq=Hq, Hkv=Hkv, D=D, L=max(pls), dtype="f32", seed=seed)
    a = gen_attention_inputs(cfg, T, prefix_lens=pls, lcap=max(pls) + T + 3)
    rng = rng_for(seed, 12)
    tokens = rng.integers(0, 1000, (B, T)).astype(np.int32)
    return st, a, tokens, rng


def _causal(q_vec, kc, vc, b, g, n_rows, scale):
    K = kc[b, g, :n_rows].astype(np.float64)
    V = vc[b, g, :n_rows].astype(np.float64)
    s = K @ q_vec.astype(np.float64) * scale
    w = np.exp(s - s.max())
    return (w[:, None] * V).sum(0) / w.sum()


@pytest.mark.parametrize("tree,Hq,Hkv", [("c0", 4, 2), ("c1", 2, 1), ("c3", 3, 3)])
def test_committed_cache_reproduces_tree_attention_causally(tree, Hq, Hkv):
    B, D = 3, 8
    st, a, tokens, rng = _setup(tree, B, Hq, Hkv, D, [4, 0, 9], seed=31)
    out = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "f32", a["prefix_len"],
                                st["mask"], Hkv)
    P = len(st["paths"])
    best = rng.integers(0, P, B).astype(np.int32)
    alen = np.array([st["path_len"][p] for p in best], np.int32)      # whole paths accepted
    alen[1] = max(0, alen[1] - 1)
    res = oracle.commit(st, best, alen, tokens, np.zeros(B, np.int32), a["k_cache"], a["v_cache"],
                        a["prefix_len"])
    scale = 1 / np.sqrt(D)
    for b in range(B):
        L = int(a["prefix_len"][b])
        path = st["paths"][best[b]]
        for hq in range(Hq):
            g = hq // (Hq // Hkv)
            for k in range(int(alen[b]) + 1):
                ref = _causal(a["q"][b, hq, path[k]], res["k_cache"], res["v_cache"], b, g,
                              L + k + 1, scale)
                np.testing.assert_allclose(out[b, hq, path[k]], ref, rtol=0, atol=1e-12)


def test_emitted_tokens_follow_parent_pointers_and_prefix_grows():
    st, a, tokens, rng = _setup("c4", 4, 2, 2, 8, [5, 6, 7, 8], seed=32, K=3)
    P = len(st["paths"])
    best = rng.integers(0, P, 4).astype(np.int32)
    alen = np.array([0, 1, 2, 3], np.int32)
    nxt = np.array([11, 22, 33, 44], np.int32)
    hidden = rng.standard_normal((4, st["T"], 16)).astype(np.float32)
    res = oracle.commit(st, best, alen, tokens, nxt, a["k_cache"], a["v_cache"], a["prefix_len"],
                        hidden)
    for b in range(4):
        last = st["paths"][best[b]][alen[b]]
        chain = []
        n = last
        while n != -1:                      # walk up to the root
            chain.append(n)
            n = st["parent"][n]
        chain.reverse()
        assert len(chain) == alen[b] + 1 == res["out_count"][b]
        assert res["out_tokens"][b, :alen[b] + 1].tolist() == [int(tokens[b][n]) for n in chain]
        assert (res["out_tokens"][b, alen[b] + 1:] == -1).all()
        assert res["prefix_len"][b] == a["prefix_len"][b] + alen[b] + 1
        assert res["new_root"][b] == nxt[b]
        assert np.array_equal(res["next_hidden"][b], hidden[b, last])


def test_rows_outside_the_destinations_are_untouched():
    st, a, tokens, rng = _setup("c1", 2, 2, 2, 8, [6, 3], seed=33, K=4)
    P = len(st["paths"])
    best = np.array([P - 1, 0], np.int32)
    alen = np.array([st["path_len"][P - 1], 0], np.int32)
    res = oracle.commit(st, best, alen, tokens, np.zeros(2, np.int32), a["k_cache"], a["v_cache"],
                        a["prefix_len"])
    for b in range(2):
        L, A = int(a["prefix_len"][b]), int(alen[b])
        keep = [r for r in range(a["k_cache"].shape[2]) if not (L + 1 <= r <= L + A)]
        assert np.array_equal(res["k_cache"][b][:, keep], a["k_cache"][b][:, keep])
        assert np.array_equal(res["v_cache"][b][:, keep], a["v_cache"][b][:, keep])
    assert np.array_equal(res["k_cache"][1], a["k_cache"][1])      # accept length 0: nothing moves


def test_leftmost_chain_is_already_in_place():
    """On a chain (every node's only child has the next id) the accepted rows are already where
    the commit puts them, so the cache is unchanged."""
    st, a, tokens, rng = _setup(cartesian_choices([1] * 6), 1, 2, 1, 4, [10], seed=34, topk=1,
                                K=6)
    res = oracle.commit(st, np.array([0], np.int32), np.array([6], np.int32), tokens,
                        np.zeros(1, np.int32), a["k_cache"], a["v_cache"], a["prefix_len"])
    assert np.array_equal(res["k_cache"], a["k_cache"])
    assert res["out_tokens"][0].tolist() == [int(t) for t in tokens[0]]
