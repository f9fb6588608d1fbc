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
    (cartesian_choices([63, 64]), 2, 64),          # T = 4096, the largest tree: 64 mask words
])
def test_edge_trees(choices, K, topk):
    _check_tree(choices, K, topk, 3, seed=K * 11 + topk)


@pytest.mark.parametrize("ci,packed,tree_name,K,topk,prefix", [
    (0, False, "c0", 3, 3, None),          # fp32, a head (the third) that fills no depth
    (1, True, "c1", 4, 10, None),
    (2, True, "c2", 5, 10, None),
    (3, True, "c3", 3, 10, [2048, 0, 7, 1999, 64, 1, 512, 1024]),
    (-1, True, "chain8", 8, 1, [5, 9]),    # every head fills one depth, topk 1
    (-2, False, "full64", 1, 64, [3]),     # one head, 64 children of the root
])
def test_fused_heads_tree_matches_heads_then_build_tree(ci, packed, tree_name, K, topk, prefix):
    """medusa_heads_build_tree (the gather done by the top-k merge) against medusa_heads
    followed by build_tree, bit for bit, and the tokens against the oracle's gather."""
    import torch
    from synth import gen_head_inputs, get_config
    from synth.configs import custom
    m = lib()
    if ci >= 0:
        cfg = get_config(ci)
        choices = load_tree_choices(tree_name)
    elif tree_name == "chain8":
        cfg = custom(dtype="bf16", B=2, Hd=256, V=700, K=8, topk=1, w_std=1 / 16, seed=81)
        choices = cartesian_choices([1] * 8)
    else:
        cfg = custom(dtype="f32", B=1, Hd=64, V=300, K=1, topk=64, w_std=1 / 8, seed=82)
        choices = cartesian_choices([64])
    B = cfg.B
    pl = np.asarray(prefix if prefix is not None else [cfg.L] * B, np.int32)
    rng = rng_for(cfg.seed, 13)
    root = rng.integers(0, cfg.V, B).astype(np.int32)
    hin = gen_head_inputs(cfg)
    w1, w2 = dev(hin["w1"]), dev(hin["w2"])
    if packed:
        w1, w2 = m.pack_weights(w1), m.pack_weights(w2)
    h, b1 = dev(hin["h"]), dev(hin["b1"])
    st = oracle.build_static(choices, topk, K)
    tree = m.Tree(choices, K, topk)
    T = st["T"]
    ws = m.workspace(m.medusa_heads_workspace(B, cfg.Hd, cfg.V, K, topk))
    out = {}
    for fused in (False, True):
        ids = torch.full((B, K, topk), -1, dtype=torch.int32, device="cuda")
        tl = torch.zeros((B, K, topk), dtype=torch.float32, device="cuda")
        lg = torch.zeros((B, K, cfg.V), dtype=torch.float32, device="cuda")
        tk = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
        ps = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
        say("fused heads + tree", tree_name, "fused" if fused else "separate")
        if not fused:
            if packed:
                m.medusa_heads_packed(h, w1, b1, w2, cfg.V, K, topk, ids, ws, logits=lg,
                                      topk_logits=tl)
            else:
                m.medusa_heads(h, w1, b1, w2, topk, ids, ws, logits=lg, topk_logits=tl)
            m.build_tree(tree, ids, dev(root), dev(pl), tk, ps)
        else:
            m.medusa_heads_build_tree(h, w1, b1, w2, cfg.V, K, topk, tree, dev(root), dev(pl), ids,
                                      tk, ps, ws, logits=lg, topk_logits=tl)
        torch.cuda.synchronize()
        out[fused] = [host(x) for x in (ids, tl, lg, tk, ps)]
    for a, b in zip(out[False], out[True]):
        assert np.array_equal(a, b)
    tokens, pos = oracle.gather(st, out[True][0], root, pl)
    assert out[True][3].tolist() == tokens and out[True][4].tolist() == pos
