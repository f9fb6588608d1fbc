"""Pins for the oracle's tree attention.

Brute force: every root-to-leaf path of a small tree is run as plain causal attention over
[prefix; root; n1; ...; nd] (Wiblog page, tree-attention section: within one path the tokens
follow the causal mask, different paths cannot see each other), and each node's output must match
the tree-masked result.  Plus textbook special cases of softmax attention.
"""

import numpy as np
import pytest

import oracle
from synth.configs import custom
from synth.gen import gen_attention_inputs, rng_for
from synth.trees import cartesian_choices, load_tree_choices


def _causal_path_attention(q, kc, vc, b, hq, g, L, path_nodes, scale):
    """Plain causal attention over the sequence prefix + path, returns one vector per path node."""
    rows = list(range(L)) + [L + n for n in path_nodes]
    K = kc[b, g, rows].astype(np.float64)
    Vv = vc[b, g, rows].astype(np.float64)
    outs = []
    for t, n in enumerate(path_nodes):
        s = K[:L + t + 1] @ q[b, hq, n].astype(np.float64) * scale
        w = np.exp(s - s.max())
        outs.append((w[:, None] * Vv[:L + t + 1]).sum(0) / w.sum())
    return outs


@pytest.mark.parametrize("tree,Hq,Hkv,L", [("c0", 4, 2, 5), ("c1", 2, 1, 3), ("c0", 3, 3, 0)])
def test_matches_per_path_causal_attention(tree, Hq, Hkv, L):
    choices = load_tree_choices(tree)
    st = oracle.build_static(choices, 10, 5)
    T = st["T"]
    cfg = custom(B=2, Hq=Hq, Hkv=Hkv, D=8, L=L, dtype="f32", seed=21)
    a = gen_attention_inputs(cfg, T, prefix_lens=[L, L + 2] if L else [0, 1])
    out = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "f32", a["prefix_len"],
                                st["mask"], Hkv)
    scale = 1 / np.sqrt(8)
    for b in range(2):
        Lb = int(a["prefix_len"][b])
        for hq in range(Hq):
            g = hq // (Hq // Hkv)
            for p, row in enumerate(st["paths"]):
                nodes = row[:st["path_len"][p] + 1]
                ref = _causal_path_attention(a["q"], a["k_cache"], a["v_cache"], b, hq, g, Lb,
                                             nodes, scale)
                for n, r in zip(nodes, ref):
                    np.testing.assert_allclose(out[b, hq, n], r, rtol=0, atol=1e-12)


def test_root_without_prefix_returns_its_own_value():
    st = oracle.build_static(cartesian_choices([2, 2]), 2, 2)
    cfg = custom(B=1, Hq=2, Hkv=2, D=16, L=0, seed=3)
    a = gen_attention_inputs(cfg, st["T"], prefix_lens=[0])
    out = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "f32", a["prefix_len"],
                                st["mask"], 2)
    for hq in range(2):
        assert np.array_equal(out[0, hq, 0], a["v_cache"][0, hq, 0].astype(np.float64))


def test_zero_query_gives_mean_of_visible_values():
    st = oracle.build_static(load_tree_choices("c0"), 3, 2)
    cfg = custom(B=1, Hq=2, Hkv=1, D=8, L=6, seed=4)
    a = gen_attention_inputs(cfg, st["T"])
    q = np.zeros_like(a["q"])
    out = oracle.tree_attention(q, a["k_cache"], a["v_cache"], "f32", a["prefix_len"],
                                st["mask"], 1)
    for i in range(st["T"]):
        vis = list(range(6)) + [6 + j for j in range(st["T"]) if (st["mask"][i][0] >> j) & 1]
        ref = a["v_cache"][0, 0, vis].astype(np.float64).mean(0)
        np.testing.assert_allclose(out[0, 1, i], ref, rtol=0, atol=1e-14)


def test_one_dominant_key_selects_its_value():
    st = oracle.build_static(load_tree_choices("c0"), 3, 2)
    T = st["T"]
    cfg = custom(B=1, Hq=1, Hkv=1, D=4, L=3, seed=5)
    a = gen_attention_inputs(cfg, T)
    kc = a["k_cache"].copy()
    kc[:] = 0
    kc[0, 0, 1, 0] = 1.0                         # prefix row 1 is the only key with any score
    q = np.zeros_like(a["q"])
    q[..., 0] = 400.0                            # score 200 vs 0: weight ratio e^-200
    out = oracle.tree_attention(q, kc, a["v_cache"], "f32", a["prefix_len"], st["mask"], 1)
    for i in range(T):
        np.testing.assert_allclose(out[0, 0, i], a["v_cache"][0, 0, 1], rtol=0, atol=1e-80)


def test_permuting_prefix_rows_changes_nothing():
    st = oracle.build_static(load_tree_choices("c0"), 3, 2)
    cfg = custom(B=1, Hq=2, Hkv=2, D=8, L=9, seed=6)
    a = gen_attention_inputs(cfg, st["T"])
    perm = rng_for(1, 1).permutation(9)
    kc, vc = a["k_cache"].copy(), a["v_cache"].copy()
    kc[:, :, :9] = kc[:, :, perm]
    vc[:, :, :9] = vc[:, :, perm]
    o1 = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "f32", a["prefix_len"],
                               st["mask"], 2)
    o2 = oracle.tree_attention(a["q"], kc, vc, "f32", a["prefix_len"], st["mask"], 2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def test_selected_units_match_full_run():
    st = oracle.build_static(load_tree_choices("c1"), 10, 4)
    cfg = custom(B=2, Hq=4, Hkv=2, D=16, L=7, dtype="bf16", seed=8)
    a = gen_attention_inputs(cfg, st["T"])
    full = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "bf16", a["prefix_len"],
                                 st["mask"], 2)
    sel = np.array([[0, 0, 0], [1, 3, 64], [1, 2, 17]])
    part = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "bf16", a["prefix_len"],
                                 st["mask"], 2, sel=sel)
    for b, h, i in sel:
        assert np.array_equal(part[b, h, i], full[b, h, i])
    assert np.isnan(part[0, 1, 1]).all()
