"""Pins for the oracle's rotary embedding at tree depth positions.

Wiblog "Medusa multi-head speculative decoding", tree-attention section: the position encoding
must give every tree token its correct position index, the one it would have when its own path
is decoded one token at a time.  So the main pin runs every root-to-leaf path as plain causal
attention over [prefix; path] with each token rotated at its sequential position (the prefix keys
rotated when "written", at 0..L-1) and requires the tree result for every node on the path.
Closed forms fix the pairing of dimensions and the frequencies; rotation invariants catch sign
and angle slips.
"""

import numpy as np
import pytest

import oracle
from oracle import bf16
from oracle.rope import rope
from synth.configs import custom
from synth.gen import gen_attention_inputs, rng_for
from synth.trees import load_tree_choices


def test_position_zero_is_the_identity():
    x = rng_for(1, 20).standard_normal((3, 5, 64))
    assert np.array_equal(rope(x, np.zeros((3, 5))), x)


def test_closed_forms_fix_pairing_and_frequencies():
    e0 = np.array([1.0, 0, 0, 0])
    e1 = np.array([0, 1.0, 0, 0])
    # dimension 0 turns with dimension D/2 = 2 at angle pos * 1
    np.testing.assert_allclose(rope(e0, 1.0), [np.cos(1), 0, np.sin(1), 0], atol=1e-15)
    # dimension 1 turns with dimension 3 at angle pos * base^(-2/4): base 100, pos 10 -> 1 rad
    np.testing.assert_allclose(rope(e1, 10.0, base=100.0), [0, np.cos(1), 0, np.sin(1)],
                               atol=1e-15)
    # a quarter turn: (a, b) -> (-b, a)
    np.testing.assert_allclose(rope(np.array([0.3, -0.7]), np.pi / 2), [0.7, 0.3], atol=1e-15)


def test_rotation_invariants():
    rng = rng_for(2, 20)
    x = rng.standard_normal((7, 128))
    p1, p2 = rng.integers(0, 9000, 7).astype(float), rng.integers(0, 9000, 7).astype(float)
    y = rope(x, p1)
    half = 64
    np.testing.assert_allclose(y[:, :half] ** 2 + y[:, half:] ** 2,
                               x[:, :half] ** 2 + x[:, half:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(rope(y, p2), rope(x, p1 + p2), atol=1e-9)
    # scores depend only on the distance between the two positions
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m_, n_, s_ in [(5, 3, 100), (4000, 17, 2222), (0, 8000, 7)]:
        a = rope(q, m_) @ rope(k, n_)
        b = rope(q, m_ + s_) @ rope(k, n_ + s_)
        assert abs(a - b) < 1e-9


@pytest.mark.parametrize("tree,Hq,Hkv,L", [("c0", 4, 2, 5), ("c1", 2, 1, 3), ("c2", 2, 2, 0)])
def test_tree_rope_matches_sequential_decoding_of_each_path(tree, Hq, Hkv, L):
    D = 16
    st = oracle.build_static(load_tree_choices(tree), 10, 5)
    T = st["T"]
    pls = [L, L + 4]
    cfg = custom(B=2, Hq=Hq, Hkv=Hkv, D=D, L=max(pls), dtype="f32", seed=23)
    a = gen_attention_inputs(cfg, T, prefix_lens=pls)
    kraw = a["k_cache"].astype(np.float64)
    kc = a["k_cache"].copy()
    for b in range(2):                      # prefix keys were rotated when they were written
        Lb = pls[b]
        kc[b, :, :Lb] = rope(kraw[b, :, :Lb], np.arange(Lb)[None, :]).astype(np.float32)
    pos = np.array([[pls[b] + d for d in st["depth"]] for b in range(2)])
    out, kr = oracle.tree_attention_rope(a["q"], kc, a["v_cache"], "f32", a["prefix_len"],
                                         st["mask"], Hkv, pos)
    scale = 1 / np.sqrt(D)
    for b in range(2):
        Lb = pls[b]
        assert np.array_equal(kr[b, :, :Lb], kc[b, :, :Lb])          # prefix untouched
        for hq in range(Hq):
            g = hq // (Hq // Hkv)
            for p, row in enumerate(st["paths"]):
                nodes = row[:st["path_len"][p] + 1]
                keys = [kc[b, g, j].astype(np.float64) for j in range(Lb)]
                keys += [rope(kraw[b, g, Lb + n], Lb + t) for t, n in enumerate(nodes)]
                vals = [a["v_cache"][b, g, j] for j in range(Lb)] + \
                       [a["v_cache"][b, g, Lb + n] for n in nodes]
                K, V = np.array(keys), np.array(vals, np.float64)
                for t, n in enumerate(nodes):
                    qv = rope(a["q"][b, hq, n].astype(np.float64), Lb + t)
                    s = K[:Lb + t + 1] @ qv * scale
                    w = np.exp(s - s.max())
                    ref = (w[:, None] * V[:Lb + t + 1]).sum(0) / w.sum()
                    # the oracle rounds rotated q and k to fp32 before attending
                    np.testing.assert_allclose(out[b, hq, n], ref, rtol=0, atol=2e-6)


def test_rotate_tree_touches_only_tree_rows_and_rounds_bf16():
    st = oracle.build_static(load_tree_choices("c1"), 10, 4)
    T = st["T"]
    cfg = custom(B=2, Hq=2, Hkv=1, D=32, L=9, dtype="bf16", seed=24)
    a = gen_attention_inputs(cfg, T, prefix_lens=[9, 2], lcap=9 + T + 6)
    pos = np.array([[9 + d for d in st["depth"]], [2 + d for d in st["depth"]]])
    qr, kr = oracle.rotate_tree(a["q"], a["k_cache"], "bf16", a["prefix_len"], pos)
    assert qr.dtype == np.uint16 and kr.dtype == np.uint16
    for b, L in enumerate([9, 2]):
        assert np.array_equal(kr[b, :, :L], a["k_cache"][b, :, :L])
        assert np.array_equal(kr[b, :, L + T:], a["k_cache"][b, :, L + T:])
        # the root (depth 0) turns by prefix_len radians-per-frequency, so it changes unless L = 0
        assert not np.array_equal(kr[b, :, L], a["k_cache"][b, :, L])
    # the rotated values are rounded once from fp64 to the nearest bf16 (ties to even), which the
    # pinned rounding of oracle/bf16.py gives; a truncating rounder would differ on many elements
    q64 = bf16.decode(a["q"])
    exact = oracle.rope(q64, pos[:, None, :])
    assert np.array_equal(qr, bf16.round_rne(exact))
    trunc = (exact.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.mean(qr != trunc) > 0.2
    # every rotated value is within half a bf16 step (2^-8 relative) of the exact rotation
    back = bf16.decode(qr)
    assert np.all(np.abs(back - exact) <= np.abs(exact) * 2.0 ** -8 + 2.0 ** -133)
    for b, L in enumerate([9, 2]):
        rows = bf16.decode(a["k_cache"][b, :, L:L + T])
        want = bf16.round_rne(oracle.rope(rows, pos[b][None, :]))
        assert np.array_equal(kr[b, :, L:L + T], want)
