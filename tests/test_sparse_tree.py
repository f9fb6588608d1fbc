"""The library's sparse-tree construction (host code, no GPU) against the oracle: the same choice
list and the same expectation, bit for bit (both take products in depth order and sum in node
order), including exact ties; invalid arguments are rejected."""

import ctypes

import numpy as np
import pytest

import oracle.sparse_tree as ost
from synth.gen import rng_for


@pytest.fixture(scope="module")
def m():
    import medusa_head_speculative_amd as m
    m.load()
    return m


def _acc(seed, K, topk, ties=False):
    rng = rng_for(seed, 31)
    if ties:
        a = rng.integers(1, 4, (K, topk)) / 8.0           # few distinct values: many exact ties
    else:
        a = rng.random((K, topk))
        a = a / a.sum(1, keepdims=True) * rng.uniform(0.4, 0.99, (K, 1))
    return a


@pytest.mark.parametrize("K,topk,N,ties", [(1, 1, 1, False), (1, 7, 7, False), (2, 3, 12, False),
                                           (3, 10, 64, False), (4, 10, 64, True),
                                           (5, 4, 300, True), (3, 6, 258, False),
                                           (8, 2, 100, True)])
def test_matches_the_oracle(m, K, topk, N, ties):
    acc = _acc(K * 100 + topk, K, topk, ties)
    got, e = m.sparse_tree(acc, N)
    ref, e_ref = ost.sparse_tree(acc.tolist(), N)
    assert got == ref
    assert e == e_ref


@pytest.mark.parametrize("K,N", [(4, 64), (5, 64), (3, 128)])
def test_synthetic_accuracy_model(m, K, N):
    acc = np.array([[0.6 * (r + 1) ** -2.35 for r in range(10)]] * K)
    got, e = m.sparse_tree(acc, N)
    ref, e_ref = ost.sparse_tree(acc.tolist(), N)
    assert got == ref and e == e_ref


def test_certain_children_and_the_full_tree(m):
    acc = np.array([[0.5, 0.3], [1.0, 0.0], [1.0, 1.0]])
    for N in range(1, 15):
        got, e = m.sparse_tree(acc, N)
        ref, e_ref = ost.sparse_tree(acc.tolist(), N)
        assert got == ref and e == e_ref


def test_invalid_arguments(m):
    L = m.load()
    out = np.zeros((10, 3), np.int32)
    acc = np.full((3, 2), 0.5)
    assert L.medusa_sparse_tree(acc.ctypes.data, 3, 2, 15, out.ctypes.data, None) == -2  # 14 nodes
    assert L.medusa_sparse_tree(acc.ctypes.data, 0, 2, 1, out.ctypes.data, None) == -2
    assert L.medusa_sparse_tree(acc.ctypes.data, 3, 65, 1, out.ctypes.data, None) == -2
    assert L.medusa_sparse_tree(None, 3, 2, 1, out.ctypes.data, None) == -1
    bad = acc.copy()
    bad[1, 1] = 1.5
    assert L.medusa_sparse_tree(bad.ctypes.data, 3, 2, 4, out.ctypes.data, None) == -1
    bad[1, 1] = np.nan
    assert L.medusa_sparse_tree(bad.ctypes.data, 3, 2, 4, out.ctypes.data, None) == -1
