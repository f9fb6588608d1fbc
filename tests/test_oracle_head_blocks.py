"""Pins for the oracle's multi-block / LayerNorm heads.

* One block without LayerNorm is the pinned single-block head.
* Zero-initialised blocks, any number of them and with or without LayerNorm, leave h unchanged,
  so every head reproduces the LM-head logits bit for bit: the property the Ultralytics page
  prints for one block, extended.
* Blocks chain: two blocks equal one block applied to the first block's output.
* LayerNorm closed forms: a constant vector normalises to beta; an alternating +-1 vector (mean 0,
  mean squared deviation 1) normalises to x / sqrt(1 + eps) * gamma, which fixes the biased
  variance and where eps enters.
"""

import numpy as np
import pytest

import oracle
from oracle.head_blocks import heads_blocks, layer_norm
from synth.configs import custom
from synth.gen import gen_head_inputs, rng_for


def _weights(rng, K, nb, hd, V, std=0.05):
    w1 = (rng.standard_normal((K, nb, hd, hd)) * std).astype(np.float32)
    b1 = (rng.standard_normal((K, nb, hd)) * std).astype(np.float32)
    w2 = (rng.standard_normal((K, V, hd)) * std).astype(np.float32)
    return w1, b1, w2


def test_one_block_without_layernorm_is_the_single_block_head():
    cfg = custom(dtype="f32", B=2, Hd=64, V=50, K=3, seed=41)
    hin = gen_head_inputs(cfg)
    r1, l1 = oracle.heads(hin["h"], hin["w1"], hin["b1"], hin["w2"], "f32")
    r2, l2 = heads_blocks(hin["h"], hin["w1"][:, None], hin["b1"][:, None], hin["w2"], "f32")
    np.testing.assert_allclose(r2, r1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nb,ln", [(1, False), (3, False), (2, True)])
def test_zero_initialised_blocks_reproduce_the_lm_head(nb, ln):
    rng = rng_for(42, 40)
    K, hd, V = 3, 32, 40
    h = rng.standard_normal((2, hd)).astype(np.float32)
    lm = (rng.standard_normal((V, hd)) * 0.02).astype(np.float32)
    w1 = np.zeros((K, nb, hd, hd), np.float32)
    b1 = np.zeros((K, nb, hd), np.float32)
    w2 = np.stack([lm] * K)
    g = rng.standard_normal((K, nb, hd)).astype(np.float32) if ln else None
    b = rng.standard_normal((K, nb, hd)).astype(np.float32) if ln else None
    _, logits = heads_blocks(h, w1, b1, w2, "f32", g, b)
    base = oracle.project(lm, "f32", h.astype(np.float64))
    for k in range(K):
        assert np.array_equal(logits[:, k], base)


@pytest.mark.parametrize("ln", [False, True])
def test_blocks_chain(ln):
    rng = rng_for(43, 40)
    K, hd, V = 2, 48, 30
    h = rng.standard_normal((3, hd)).astype(np.float32)
    w1, b1, w2 = _weights(rng, K, 2, hd, V)
    g = rng.uniform(0.5, 1.5, (K, 2, hd)).astype(np.float32) if ln else None
    b = (rng.standard_normal((K, 2, hd)) * 0.1).astype(np.float32) if ln else None
    r2, l2 = heads_blocks(h, w1, b1, w2, "f32", g, b)
    for k in range(K):
        sl = slice(k, k + 1)
        r1, _ = heads_blocks(h, w1[sl, :1], b1[sl, :1], w2[sl], "f32",
                             None if g is None else g[sl, :1], None if b is None else b[sl, :1])
        rr, ll = heads_blocks(r1[:, 0], w1[sl, 1:], b1[sl, 1:], w2[sl], "f32",
                              None if g is None else g[sl, 1:], None if b is None else b[sl, 1:])
        np.testing.assert_allclose(rr[:, 0], r2[:, k], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ll[:, 0], l2[:, k], rtol=0, atol=1e-12)


def test_layernorm_closed_forms():
    hd, eps = 8, 1e-5
    gamma, beta = np.full(hd, 2.0), np.linspace(-1, 1, hd)
    np.testing.assert_allclose(layer_norm(np.full((1, hd), 3.7), gamma, beta, eps)[0], beta,
                               atol=1e-15)
    x = np.array([[1.0, -1.0] * (hd // 2)])
    np.testing.assert_allclose(layer_norm(x, gamma, np.zeros(hd), eps)[0],
                               2.0 * x[0] / np.sqrt(1.0 + eps), rtol=1e-15)
    # through a whole head: W1 = I, b1 = 0, so r = x + SiLU(LN(x))
    w1 = np.eye(hd, dtype=np.float32)[None, None]
    b1 = np.zeros((1, 1, hd), np.float32)
    w2 = np.eye(hd, dtype=np.float32)[None]
    g = np.full((1, 1, hd), 2.0, np.float32)
    z = np.zeros((1, 1, hd), np.float32)
    r, logits = heads_blocks(x.astype(np.float32), w1, b1, w2, "f32", g, z)
    u = 2.0 * x[0] / np.sqrt(1.0 + eps)
    np.testing.assert_allclose(r[0, 0], x[0] + u / (1 + np.exp(-u)), rtol=1e-15)
    np.testing.assert_allclose(logits[0, 0], r[0, 0], rtol=1e-15)
