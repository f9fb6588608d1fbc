"""GPU parity of evaluate_posterior (the page's candidate-filtering call with its top_p,
sampling and fast arguments) against the fp64 oracle, through the C ABI.

Nucleus decisions whose mass above the candidate lies within 1e-4 (relative, |ln top_p -
ln mass|) of top_p may go either way between fp64 and fp32; the GPU result must then equal one of
the results obtained by flipping them."""

import numpy as np
import pytest

import oracle
from gpu_util import accept_candidates, dev, host, lib, say
from synth import gen_verif_logits, get_config
from synth.configs import custom
from synth.gen import rng_for
from synth.trees import cartesian_choices, load_tree_choices

pytestmark = pytest.mark.gpu


def _tree_and_tokens(m, choices, K, topk, B, V, seed):
    import torch
    st = oracle.build_static(choices, topk, K)
    tree = m.Tree(choices, K, topk)
    rng = rng_for(seed, 11)
    ids = np.stack([np.stack([rng.choice(V, size=topk, replace=False) for _ in range(K)])
                    for _ in range(B)]).astype(np.int32)
    root = rng.integers(0, V, B).astype(np.int32)
    tokens, _ = oracle.gather(st, ids, root, [0] * B)
    tt = torch.zeros((B, st["T"]), dtype=torch.int32, device="cuda")
    pp = torch.zeros((B, st["T"]), dtype=torch.int32, device="cuda")
    m.build_tree(tree, dev(ids), dev(root), dev(np.zeros(B, np.int32)), tt, pp)
    return st, tree, np.array(tokens, np.int32)


def run_posterior(m, tree, logits, tokens, temp, top_p, sampling, fast=False, eps=0.09,
                  delta=0.3):
    import torch
    B = logits.shape[0]
    ws = m.workspace(m.evaluate_posterior_workspace(B, logits.shape[2], tree, sampling))
    outs = [torch.full((B,), -1, dtype=torch.int32, device="cuda") for _ in range(3)]
    m.evaluate_posterior(dev(logits), dev(tokens), tree, temp, eps, delta, outs[0], outs[1], ws,
                         top_p=top_p, sampling=sampling, fast=fast, next_token=outs[2])
    torch.cuda.synchronize()
    return tuple(host(o) for o in outs)


def _check(st, res, logits, dtype, got):
    cands, nband = accept_candidates(st, res, logits, dtype)
    for b in range(len(cands)):
        assert (int(got[0][b]), int(got[1][b]), int(got[2][b])) in cands[b], (b, got, cands[b])
    return nband


@pytest.mark.parametrize("ci,top_p", [(0, 0.9), (1, 0.5), (1, 0.95), (2, 0.9), (3, 0.8),
                                      (4, 0.9), (4, 0.99)])
def test_nucleus_full_size(ci, top_p):
    cfg = get_config(ci)
    m = lib()
    temp = 0.7
    st, tree, tokens = _tree_and_tokens(m, load_tree_choices(f"c{ci}"), cfg.K, cfg.topk, cfg.B,
                                        cfg.V, seed=ci + 50)
    logits = gen_verif_logits(cfg, st["parent"], tokens, seed=ci + 50)
    res = oracle.evaluate_posterior(logits, cfg.dtype, tokens, st, float(np.float32(temp)),
                                    top_p=float(np.float32(top_p)), sampling="nucleus")
    say("nucleus full size", cfg.name, top_p)
    got = run_posterior(m, tree, logits, tokens, temp, top_p, "nucleus")
    nband = _check(st, res, logits, cfg.dtype, got)
    acc = int(res["accepted"][:, 1:].sum())
    print(f"{cfg.name} top_p={top_p}: accept_length {got[1].tolist()} oracle "
          f"{res['accept_length'].tolist()}, {acc} of {cfg.B * (st['T'] - 1)} candidates in the "
          f"nucleus, banded {nband}")
    # the fast flag changes nothing, bit for bit
    got2 = run_posterior(m, tree, logits, tokens, temp, top_p, "nucleus", fast=True)
    assert all(np.array_equal(x, y) for x, y in zip(got, got2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,tree,B,temp,top_p", [
    (1, "one", 1, 0.7, 0.5), (7, "c0", 2, 1.0, 0.6), (2047, "c1", 3, 0.3, 0.9),
    (5000, "chain6", 2, 2.0, 0.7), (4100, "c3", 5, 0.7, 0.3), (20001, "c4", 3, 0.7, 0.95),
    (131077, "chain8", 4, 1.0, 0.8),
])
def test_nucleus_edges(dtype, V, tree, B, temp, top_p):
    m = lib()
    if tree == "one":
        choices, K, topk = [[0]], 1, 1
    elif tree in ("chain6", "chain8"):
        depth = int(tree[5:])
        choices, K, topk = cartesian_choices([1] * depth), depth, 1
    else:
        choices, K, topk = load_tree_choices(tree), 5, 10
    topk = min(topk, V)
    choices = [c for c in choices if max(c) < topk]
    st, tr, tokens = _tree_and_tokens(m, choices, K, topk, B, V, seed=V + B + 7)
    cfg = custom(dtype=dtype, B=B, V=V, seed=V * 5 + B, boost_p=0.8)
    logits = gen_verif_logits(cfg, st["parent"], tokens)
    res = oracle.evaluate_posterior(logits, dtype, tokens, st, float(np.float32(temp)),
                                    top_p=float(np.float32(top_p)), sampling="nucleus")
    say("nucleus edge", dtype, V, tree, B, temp, top_p)
    _check(st, res, logits, dtype, run_posterior(m, tr, logits, tokens, temp, top_p, "nucleus"))


def test_nucleus_limits_and_typical_mode():
    """top_p = 1: every finite candidate is in; a tiny top_p: only the row maxima, the greedy
    decisions; temperature 0: greedy in both modes; sampling = typical: typical_accept bit for
    bit."""
    import torch
    m = lib()
    cfg = get_config(1)
    st, tree, tokens = _tree_and_tokens(m, load_tree_choices("c1"), 4, 10, 2, cfg.V, seed=71)
    # make some children their parent row's argmax, so the greedy walk goes somewhere
    logits = gen_verif_logits(custom(dtype="bf16", B=2, V=cfg.V, seed=71, boost=40.0, boost_p=0.5),
                              st["parent"], tokens)
    say("nucleus limits")
    full = run_posterior(m, tree, logits, tokens, 0.7, 1.0, "nucleus")
    assert full[1].tolist() == [max(st["path_len"])] * 2
    greedy = oracle.typical_accept(logits, "bf16", tokens.tolist(), st, 0.0)
    tiny = run_posterior(m, tree, logits, tokens, 0.7, 1e-9, "nucleus")
    res = oracle.evaluate_posterior(logits, "bf16", tokens.tolist(), st, float(np.float32(0.7)),
                                    top_p=float(np.float32(1e-9)), sampling="nucleus")
    _check(st, res, logits, "bf16", tiny)
    # (equal to greedy unless two candidates tie at a row's maximum, when both are in)
    g0 = run_posterior(m, tree, logits, tokens, 0.0, 0.5, "nucleus")
    assert g0[1].tolist() == greedy["accept_length"].tolist()
    assert g0[0].tolist() == greedy["best_candidate"].tolist()
    typ = run_posterior(m, tree, logits, tokens, 0.7, 0.5, "typical")
    ws = m.workspace(m.typical_accept_workspace(2, st["T"], cfg.V, tree.dims["n_internal"]))
    ref = [torch.full((2,), -1, dtype=torch.int32, device="cuda") for _ in range(3)]
    m.typical_accept(dev(logits), dev(tokens), tree, 0.7, 0.09, 0.3, ref[0], ref[1], ws,
                     next_token=ref[2])
    torch.cuda.synchronize()
    assert all(np.array_equal(x, host(y)) for x, y in zip(typ, ref))
    print(f"top_p=1 accept_length {full[1].tolist()}, tiny top_p {tiny[1].tolist()}, "
          f"greedy {greedy['accept_length'].tolist()}")


@pytest.mark.parametrize("ci,nseeds", [(0, 16), (1, 16), (2, 8)])
def test_nucleus_seed_sweep(ci, nseeds):
    """The nucleus mode over fresh tree tokens and verification logits per seed, top_p cycling
    through 0.5, 0.8, 0.9 and 0.95, temperature 0.7: every result equals the oracle's up to the
    decisions inside the 1e-4 band, whose number is bounded (at most 1 in 500, and at least 2)."""
    cfg = get_config(ci)
    m = lib()
    choices = load_tree_choices(f"c{ci}")
    banded = decisions = 0
    for j in range(nseeds):
        seed = 300 + j
        top_p = (0.5, 0.8, 0.9, 0.95)[j % 4]
        st, tree, tokens = _tree_and_tokens(m, choices, cfg.K, cfg.topk, cfg.B, cfg.V, seed=seed)
        logits = gen_verif_logits(cfg, st["parent"], tokens, seed=seed)
        res = oracle.evaluate_posterior(logits, cfg.dtype, tokens, st, float(np.float32(0.7)),
                                        top_p=float(np.float32(top_p)), sampling="nucleus")
        say("nucleus seed sweep", cfg.name, seed, top_p)
        banded += _check(st, res, logits, cfg.dtype,
                         run_posterior(m, tree, logits, tokens, 0.7, top_p, "nucleus"))
        decisions += cfg.B * (st["T"] - 1)
    print(f"{cfg.name}: {nseeds} seeds, banded {banded} of {decisions} decisions")
    assert banded <= max(2, decisions // 500)
