"""Pins for the oracle's sparse-tree construction.

* Brute force: over every prefix-closed N-node subset of small full trees, none has a larger
  expectation than the oracle's choice (and the choice is itself prefix-closed).
* The objective's reading: simulating the right path (each head's right candidate drawn from its
  accuracy table, or none) and measuring the accept length of the tree reproduces the
  expectation within sampling error.
* With the synthetic accuracy model fitted to the pages' 60 % / 80 % (the same for every head),
  the 64-node depth-4 choice equals the checked-in sparse tree of that workload.
"""

import itertools

import numpy as np
import pytest

from oracle.sparse_tree import all_nodes, expected_accept_length, node_prob, sparse_tree
from synth.gen import rng_for
from synth.trees import load_tree_choices


def _prefix_closed(sel):
    s = set(map(tuple, sel))
    return all(len(t) == 1 or t[:-1] in s for t in s)


def _random_acc(rng, K, topk):
    a = rng.random((K, topk))
    return (a / a.sum(1, keepdims=True) * rng.uniform(0.5, 0.95, (K, 1))).tolist()


@pytest.mark.parametrize("K,topk,N,seed", [(2, 3, 4, 1), (2, 4, 6, 2), (3, 2, 5, 3),
                                           (3, 2, 9, 4), (1, 5, 3, 5)])
def test_no_prefix_closed_tree_beats_the_choice(K, topk, N, seed):
    acc = _random_acc(rng_for(seed, 30), K, topk)
    sel, value = sparse_tree(acc, N)
    assert len(sel) == N and _prefix_closed(sel)
    best = -1.0
    for combo in itertools.combinations(all_nodes(K, topk), N):
        if _prefix_closed(combo):
            best = max(best, sum(node_prob(acc, t) for t in combo))
    assert abs(best - value) <= 1e-15


def test_expectation_matches_a_simulation_of_the_right_path():
    rng = rng_for(6, 30)
    K, topk = 3, 4
    acc = np.array(_random_acc(rng, K, topk))
    sel, value = sparse_tree(acc.tolist(), 9)
    tree = set(map(tuple, sel))
    n = 200000
    # right candidate per head: rank r with probability acc[k][r], none (-1) otherwise
    right = np.full((n, K), -1)
    for k in range(K):
        u = rng.random(n)
        edges = np.cumsum(acc[k])
        right[:, k] = np.where(u < edges[-1], np.searchsorted(edges, u, side="right"), -1)
    lengths = np.zeros(n)
    for i in range(n):
        d = 0
        while d < K and right[i, d] >= 0 and tuple(right[i, :d + 1]) in tree:
            d += 1
        lengths[i] = d
    sd = lengths.std() / np.sqrt(n)
    assert abs(lengths.mean() - value) < 4 * sd, (lengths.mean(), value, sd)


def test_single_head_and_equal_accuracies():
    sel, v = sparse_tree([[0.1, 0.5, 0.2, 0.05]], 2)
    assert sel == [[1], [2]] and abs(v - 0.7) < 1e-15
    # equal accuracies: every depth-1 node beats every depth-2 node, ties go by rank tuple
    sel, _ = sparse_tree([[0.3] * 3, [0.3] * 3], 5)
    assert sel == [[0], [1], [2], [0, 0], [0, 1]]


def test_a_certain_child_ties_its_parent_and_comes_after_it():
    """Accuracy 1 makes a child exactly as likely as its parent: depth breaks the tie, which is
    what keeps the choice a tree."""
    acc = [[0.5, 0.3], [1.0, 0.0]]
    assert sparse_tree(acc, 1)[0] == [[0]]
    assert sparse_tree(acc, 2)[0] == [[0], [0, 0]]
    assert sparse_tree(acc, 3)[0] == [[0], [1], [0, 0]]


@pytest.mark.parametrize("name,N,K", [("c1", 64, 4), ("c3", 128, 3)])
def test_synthetic_accuracy_model_gives_the_checked_in_sparse_trees(name, N, K):
    acc = [[0.6 * (r + 1) ** -2.35 for r in range(10)] for _ in range(K)]
    sel, v = sparse_tree(acc, N)
    ref = load_tree_choices(name)
    assert sorted(map(tuple, sel)) == sorted(map(tuple, ref))
    assert abs(v - expected_accept_length(acc, ref)) < 1e-15
