"""Pins for the oracle's heads and top-k against facts the pages and mathematics fix.

Ultralytics "Medusa Heads", how-the-heads-predict section: zero W1/b1 with W2 copied from the LM
head reproduce the base model's next-token logits exactly (the sample prints [True, True, True]).
The other pins are closed forms of h + SiLU(W1 h + b1) followed by W2, chosen so that a dropped
residual, a bias on the wrong side of SiLU, a transposed weight, a wrong head stride or a
sigmoid in place of SiLU each fail at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from synth.gen import f32_to_bf16_bits, rng_for

pytestmark = pytest.mark.filterwarnings("ignore")


def _f32(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def test_zero_init_reproduces_lm_head(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "zero_init_heads.json")))
    hd, V, K = g["hidden_size"], g["vocab_size"], g["num_heads"]
    rng = rng_for(123, 0)
    lm = _f32(rng, (V, hd), 0.02)
    h = _f32(rng, (1, hd))
    w1 = np.zeros((K, hd, hd), np.float32)
    b1 = np.zeros((K, hd), np.float32)
    w2 = np.ascontiguousarray(np.broadcast_to(lm, (K, V, hd)))
    r, logits = oracle.heads(h, w1, b1, w2, "f32")
    base = oracle.project(lm, "f32", h.astype(np.float64))
    printed = [bool(np.array_equal(logits[:, k], base)) for k in range(K)]
    assert printed == g["printed"]
    assert np.array_equal(r[0, 0], h[0].astype(np.float64))
    # the projection itself against numpy's product (different summation order)
    ref = lm.astype(np.float64) @ h[0].astype(np.float64)
    np.testing.assert_allclose(base[0], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("c", [math.log(3.0), -math.log(3.0), 2.0])
def test_bias_goes_inside_silu(c):
    # W1 = 0, b1 = c: u = c, so r = h + c * sigmoid(c); sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    hd, K = 16, 2
    h = _f32(rng_for(5, 0), (1, hd))
    w1 = np.zeros((K, hd, hd), np.float32)
    b1 = np.full((K, hd), c, np.float32)
    w2 = np.zeros((K, 3, hd), np.float32)
    r, _ = oracle.heads(h, w1, b1, w2, "f32")
    cf = float(np.float32(c))
    sig = {math.log(3.0): 0.75, -math.log(3.0): 0.25}.get(c, 1.0 / (1.0 + math.exp(-cf)))
    expect = h[0].astype(np.float64) + cf * sig
    np.testing.assert_allclose(r[0, 0], expect, rtol=0, atol=1e-7)
    np.testing.assert_allclose(r[0, 1], expect, rtol=0, atol=1e-7)


def test_w1_is_out_by_in():
    # a single nonzero W1[k][i0][j0] = a changes output i0 only, through input j0
    hd, K, i0, j0, a = 12, 1, 3, 9, 1.5
    h = _f32(rng_for(6, 0), (1, hd))
    w1 = np.zeros((K, hd, hd), np.float32)
    w1[0, i0, j0] = a
    b1 = np.zeros((K, hd), np.float32)
    w2 = np.zeros((K, 2, hd), np.float32)
    r, _ = oracle.heads(h, w1, b1, w2, "f32")
    u = a * float(h[0, j0])
    expect = h[0].astype(np.float64).copy()
    expect[i0] += u / (1.0 + math.exp(-u))
    np.testing.assert_allclose(r[0, 0], expect, rtol=0, atol=1e-14)


def test_w2_permutation_picks_residual_entries():
    hd, V, K = 16, 40, 3
    rng = rng_for(7, 0)
    h = _f32(rng, (2, hd))
    w1 = _f32(rng, (K, hd, hd), 0.3)
    b1 = _f32(rng, (K, hd), 0.3)
    w2 = np.zeros((K, V, hd), np.float32)
    perm = [(7 * v + 3) % hd for v in range(V)]
    for k in range(K):
        for v in range(V):
            w2[k, v, perm[v]] = float(k + 1)        # head k scales by k+1: pins the head stride
    r, logits = oracle.heads(h, w1, b1, w2, "f32")
    for b in range(2):
        for k in range(K):
            assert np.array_equal(logits[b, k], (k + 1) * r[b, k, perm])


def test_scaling_w2_by_two_doubles_logits_exactly():
    hd, V, K = 32, 50, 2
    rng = rng_for(8, 0)
    h = _f32(rng, (3, hd))
    w1 = _f32(rng, (K, hd, hd), 0.2)
    b1 = _f32(rng, (K, hd), 0.2)
    w2 = _f32(rng, (K, V, hd), 0.2)
    _, l1 = oracle.heads(h, w1, b1, w2, "f32")
    _, l2 = oracle.heads(h, w1, b1, (w2 * 2).astype(np.float32), "f32")
    assert np.array_equal(l2, 2 * l1)


def test_heads_use_their_own_weights_and_batch_rows_are_independent():
    hd, V, K, B = 24, 30, 3, 3
    rng = rng_for(9, 0)
    h = _f32(rng, (B, hd))
    w1 = _f32(rng, (K, hd, hd), 0.2)
    b1 = _f32(rng, (K, hd), 0.2)
    w2 = _f32(rng, (K, V, hd), 0.2)
    r, logits = oracle.heads(h, w1, b1, w2, "f32")
    for k in range(K):
        for b in range(B):
            rk, lk = oracle.heads(h[b:b + 1].copy(), w1[k:k + 1].copy(), b1[k:k + 1].copy(),
                                  w2[k:k + 1].copy(), "f32")
            assert np.array_equal(rk[0, 0], r[b, k])
            assert np.array_equal(lk[0, 0], logits[b, k])


def test_bf16_inputs_decode_exactly():
    # bf16 bit patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3FC0 = 1.5, 0x3E80 = 0.25
    hd, V, K = 8, 4, 1
    h = np.array([[0x3F80, 0xC000, 0x3FC0, 0x3E80, 0, 0, 0, 0]], np.uint16)
    w1 = np.zeros((K, hd, hd), np.uint16)
    b1 = np.zeros((K, hd), np.uint16)
    w2 = np.zeros((K, V, hd), np.uint16)
    for v in range(V):
        w2[0, v, v] = 0x3F80
    w2[0, 3, 0] = 0xC000                       # row 3: 0.25 + (-2)*1.0
    _, logits = oracle.heads(h, w1, b1, w2, "bf16")
    assert logits[0, 0].tolist() == [1.0, -2.0, 1.5, -1.75]
    assert f32_to_bf16_bits(np.array([1.0, -2.0, 1.5, 0.25], np.float32)).tolist() == \
        [0x3F80, 0xC000, 0x3FC0, 0x3E80]


def test_topk_matches_a_full_sort_with_ties_to_lower_id():
    rng = rng_for(10, 0)
    for n, k in [(1, 1), (7, 3), (50, 10), (64, 64), (200, 13)]:
        x = rng.integers(-3, 4, size=(4, n)).astype(np.float64)    # many exact ties
        ids, vals = oracle.topk(x, k)
        for r in range(4):
            ref = sorted(range(n), key=lambda v: (-x[r, v], v))[:k]
            assert ids[r].tolist() == ref
            assert vals[r].tolist() == [x[r, v] for v in ref]


def test_topk_hand_ties():
    ids, _ = oracle.topk(np.array([[1.0, 3.0, 3.0, 2.0, 3.0]]), 3)
    assert ids.tolist() == [[1, 2, 4]]
    ids, _ = oracle.topk(np.array([[0.0, 0.0, 0.0]]), 2)
    assert ids.tolist() == [[0, 1]]


def test_topk_tie_flags():
    x = np.array([[5.0, 4.0, 3.0, 2.0], [5.0, 4.0, 4.0 - 1e-6, 1.0], [5.0, 4.0, 3.0, 3.0]])
    # k = 2 looks at ranks 0..2 (the k-1 vs k boundary included)
    assert oracle.topk_ties(x, 2).tolist() == [False, True, False]
    assert oracle.topk_ties(x, 3).tolist() == [False, True, True]
