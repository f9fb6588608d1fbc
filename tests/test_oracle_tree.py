"""Pins for the oracle's candidate tree.

Counts printed on the pages (tests/golden/tree_counts.json), the ancestor-only mask rebuilt by an
independent parent walk, and the reading position = prefix_len + depth.
"""

import itertools
import json
import os
import random

import pytest

import oracle
from oracle.tree import TreeError
from synth.trees import cartesian_choices, load_tree_choices


def test_page_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tree_counts.json")))
    for case in g["cases"]:
        ks = case["ks"]
        st = oracle.build_static(cartesian_choices(ks), max(ks), len(ks))
        assert len(st["paths"]) == case["paths"]
        assert st["dmax"] == case["depth"]
        assert st["T"] - 1 == case["nodes_without_root"]
        assert all(l == case["depth"] for l in st["path_len"])


@pytest.mark.parametrize("name,T,hist,P", [
    ("c0", 9, {1: 2, 2: 6}, 6),
    ("c1", 65, {1: 9, 2: 16, 3: 20, 4: 19}, 33),
    ("c2", 65, {1: 7, 2: 14, 3: 13, 4: 19, 5: 11}, 28),
    ("c3", 129, {1: 10, 2: 42, 3: 76}, 85),
])
def test_workload_trees(name, T, hist, P):
    st = oracle.build_static(load_tree_choices(name), 10, 5)
    assert st["T"] == T and len(st["paths"]) == P
    h = {}
    for d in st["depth"][1:]:
        h[d] = h.get(d, 0) + 1
    assert h == hist


def _walk_mask(st):
    T = st["T"]
    m = [[0] * st["W"] for _ in range(T)]
    for i in range(T):
        j = i
        while j >= 0:
            m[i][j // 64] |= 1 << (j % 64)
            j = st["parent"][j]
    return m


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_mask_is_ancestor_closure(name):
    st = oracle.build_static(load_tree_choices(name), 10, 5)
    assert st["mask"] == _walk_mask(st)
    # parents precede children; depth increases by one along each edge
    for i in range(1, st["T"]):
        assert st["parent"][i] < i
        assert st["depth"][i] == st["depth"][st["parent"][i]] + 1


def test_no_cross_branch_visibility():
    st = oracle.build_static(cartesian_choices([2, 3]), 3, 2)
    nodes = st["nodes"]
    for i, ti in enumerate(nodes):
        for j, tj in enumerate(nodes):
            bit = (st["mask"][i][j // 64] >> (j % 64)) & 1
            on_path = ti[:len(tj)] == tj
            assert bit == on_path
    # siblings at depth 2 never see each other
    a, b = nodes.index((0, 0)), nodes.index((0, 1))
    assert not (st["mask"][a][0] >> b) & 1 and not (st["mask"][b][0] >> a) & 1


def test_paths_are_parent_chains_in_rank_order():
    st = oracle.build_static(load_tree_choices("c1"), 10, 4)
    leaves = []
    for p, row in enumerate(st["paths"]):
        n = st["path_len"][p]
        assert row[0] == 0 and all(x == -1 for x in row[n + 1:])
        for d in range(1, n + 1):
            assert st["parent"][row[d]] == row[d - 1]
        assert not st["children"][row[n]]
        leaves.append(st["nodes"][row[n]])
    assert leaves == sorted(leaves)
    assert len(leaves) == sum(1 for c in st["children"] if not c)


def test_gather_tokens_and_positions_c0():
    st = oracle.build_static(cartesian_choices([2, 3]), 3, 3)
    topk = [[[11, 12, 13], [21, 22, 23], [31, 32, 33]]]
    tokens, pos = oracle.gather(st, topk, [7], [128])
    # node order: root, (0), (1), (0,0), (0,1), (0,2), (1,0), (1,1), (1,2)
    assert tokens == [[7, 11, 12, 21, 22, 23, 21, 22, 23]]
    assert pos == [[128, 129, 129, 130, 130, 130, 130, 130, 130]]


@pytest.mark.parametrize("bad,err", [
    ([[0, 0]], "no parent"),
    ([[0], [3]], "rank out of range"),
    ([[0], [0, 0], [0, 0, 0], [0, 0, 0, 0]], "exceeds head count"),
    ([[0], [0]], "duplicate"),
    ([[]], "empty"),
])
def test_malformed_choices_rejected(bad, err):
    with pytest.raises(TreeError, match=err):
        oracle.build_static(bad, 3, 3)


def test_random_prefix_closed_trees():
    rnd = random.Random(0)
    for _ in range(20):
        k, K = rnd.randint(1, 4), rnd.randint(1, 4)
        allc = [t for d in range(1, K + 1) for t in itertools.product(range(k), repeat=d)]
        pick = set()
        for t in rnd.sample(allc, rnd.randint(1, len(allc))):
            for d in range(1, len(t) + 1):
                pick.add(t[:d])
        st = oracle.build_static([list(t) for t in pick], k, K)
        assert st["T"] == len(pick) + 1
        assert st["mask"] == _walk_mask(st)
