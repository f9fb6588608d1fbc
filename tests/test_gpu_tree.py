"""GPU parity of build_tree: the static arrays the C ABI uploads and the per-step gather."""

import numpy as np
import pytest

import oracle
from gpu_util import dev, host, lib, say
from synth.gen import rng_for
from synth.trees import cartesian_choices, load_tree_choices

pytestmark = pytest.mark.gpu


def _check_tree(choices, K, topk, B, seed):
    import torch
    m = lib()
    st = oracle.build_static(choices, topk, K)
    tree = m.Tree(choices, K, topk)
    d = tree.dims
    assert (d["T"], d["W"], d["n_paths"], d["dmax"]) == (st["T"], st["W"], len(st["paths"]), st["dmax"])
    rng = rng_for(seed, 0)
    topk_ids = rng.integers(0, 50000, (B, K, topk)).astype(np.int32)
    root = rng.integers(0, 50000, B).astype(np.int32)
    pl = rng.integers(0, 9000, B).astype(np.int32)
    T = st["T"]
    tokens = torch.full((B, T), -1, dtype=torch.int32, device="cuda")
    pos = torch.full((B, T), -1, dtype=torch.int32, device="cuda")
    say("build_tree", len(choices), K, topk, B)
    m.build_tree(tree, dev(topk_ids), dev(root), dev(pl), tokens, pos)
    torch.cuda.synchronize()
    et, ep = oracle.gather(st, topk_ids, root, pl)
    assert host(tokens).tolist() == et and host(pos).tolist() == ep
    assert host(tree.mask).view(np.uint64).tolist() == [[int(w) for w in r] for r in st["mask"]]
    assert host(tree.parent).tolist() == st["parent"]
    assert host(tree.depth).tolist() == st["depth"]
    assert host(tree.paths).tolist() == st["paths"]
    assert host(tree.path_len).tolist() == st["path_len"]
    kids = host(tree.child_ptr)
    idx = host(tree.child_idx)
    for i in range(T):
        assert idx[kids[i]:kids[i + 1]].tolist() == st["children"][i]
    assert host(tree.internal).tolist() == [i for i in range(T) if st["children"][i]]
    # second call: gather only
    topk2 = (topk_ids + 1).astype(np.int32)
    m.build_tree(tree, dev(topk2), dev(root), dev(pl), tokens, pos)
    torch.cuda.synchronize()
    assert host(tokens).tolist() == oracle.gather(st, topk2, root, pl)[0]


@pytest.mark.parametrize("name,K", [("c0", 3), ("c1", 4), ("c2", 5), ("c3", 3), ("c4", 3)])
def test_workload_trees(name, K):
    _check_tree(load_tree_choices(name), K, 10, 4, seed=len(name) + K)


@pytest.mark.parametrize("choices,K,topk", [
    ([[0]], 1, 1),
    (cartesian_choices([1] * 8), 8, 1),
    (cartesian_choices([64]), 1, 64),
    (cartesian_choices([3, 3, 3, 3]), 4, 3),
    (cartesian_choices([4, 4, 4, 4, 3]), 5, 4),   # T = 1365 + ... : 22 mask words
])
def test_edge_trees(choices, K, topk):
    _check_tree(choices, K, topk, 3, seed=K * 11 + topk)
