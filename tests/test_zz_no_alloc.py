"""typical_accept_noalloc (the allocation-free variant of typical_accept, its intermediates in the
library's per-GPU scratch array) against typical_accept with a caller workspace, through the C
ABI: two calls in a row, the second smaller, so the second reads a scratch array that still holds
the first call's intermediates.  Both must also be one of the results the fp64 oracle allows."""

import numpy as np
import pytest

import oracle
from gpu_util import accept_candidates, dev, host, lib, say
from synth import gen_verif_logits
from synth.configs import custom
from synth.gen import rng_for
from synth.trees import load_tree_choices

pytestmark = pytest.mark.gpu


def _case(m, tree_name, K, topk, B, V, dtype, seed):
    choices = load_tree_choices(tree_name)
    st = oracle.build_static(choices, topk, K)
    tree = m.Tree(choices, K, topk)
    rng = rng_for(seed, 11)
    ids = np.stack([np.stack([rng.choice(V, size=topk, replace=False) for _ in range(K)])
                    for _ in range(B)]).astype(np.int32)
    root = rng.integers(0, V, B).astype(np.int32)
    tokens, _ = oracle.gather(st, ids, root, np.zeros(B, np.int32))
    tokens = np.asarray(tokens, np.int32)
    # the first build_tree uploads the tree's static arrays; its tokens must be the oracle's
    import torch
    tt = torch.zeros((B, st["T"]), dtype=torch.int32, device="cuda")
    pp = torch.zeros((B, st["T"]), dtype=torch.int32, device="cuda")
    m.build_tree(tree, dev(ids), dev(root), dev(np.zeros(B, np.int32)), tt, pp)
    torch.cuda.synchronize()
    assert np.array_equal(host(tt), tokens)
    cfg = custom(dtype=dtype, B=B, V=V, seed=seed, boost_p=0.7)
    logits = gen_verif_logits(cfg, st["parent"], tokens)
    return st, tree, tokens, logits


def _run_both(m, tree, logits, tokens, temp):
    import torch
    B, T, V = logits.shape
    lg, tk = dev(logits), dev(tokens)
    outs = []
    for noalloc in (False, True):
        best = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        alen = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            m.typical_accept_noalloc(lg, tk, tree, temp, 0.09, 0.3, best, alen, next_token=nxt)
        else:
            ws = m.workspace(m.typical_accept_workspace(B, T, V, tree.dims["n_internal"]))
            m.typical_accept(lg, tk, tree, temp, 0.09, 0.3, best, alen, ws, next_token=nxt)
        torch.cuda.synchronize()
        outs.append((host(best), host(alen), host(nxt)))
    return outs


@pytest.mark.parametrize("order", ["large_then_small", "c4_then_c0"])
def test_noalloc_matches_workspace_variant_twice(order):
    m = lib()
    if order == "large_then_small":
        cases = [("c3", 3, 10, 8, 32000, "bf16", 0.7, 31), ("c1", 4, 10, 1, 32000, "bf16", 0.7, 32)]
    else:
        cases = [("c4", 3, 10, 4, 128256, "bf16", 0.7, 41), ("c0", 3, 3, 1, 1000, "f32", 0.7, 42)]
    for tree_name, K, topk, B, V, dtype, temp, seed in cases:
        st, tree, tokens, logits = _case(m, tree_name, K, topk, B, V, dtype, seed)
        say("noalloc", order, tree_name, B, V, dtype, temp)
        ws_out, na_out = _run_both(m, tree, logits, tokens, temp)
        for a, b in zip(ws_out, na_out):
            assert np.array_equal(a, b), (tree_name, a, b)
        res = oracle.typical_accept(logits, dtype, tokens.tolist(), st, float(np.float32(temp)),
                                    float(np.float32(0.09)), float(np.float32(0.3)))
        cands, nband = accept_candidates(st, res, logits, dtype)
        for b in range(B):
            assert (int(na_out[0][b]), int(na_out[1][b]), int(na_out[2][b])) in cands[b]
        print(f"{tree_name} B={B}: accept_length {na_out[1].tolist()} banded {nband}")
