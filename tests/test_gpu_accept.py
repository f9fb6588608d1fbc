"""GPU parity of typical_accept against the fp64 oracle, through the C ABI.

Decisions within 1e-4 (relative, |ln p - ln thr|) of the threshold may go either way between fp64
and fp32; the GPU result must then equal one of the results obtained by flipping them."""

import numpy as np
import pytest

import oracle
from gpu_util import accept_candidates, dev, host, lib, say
from synth import gen_verif_logits, get_config
from synth.configs import custom
from synth.gen import rng_for
from synth.trees import cartesian_choices, load_tree_choices

pytestmark = pytest.mark.gpu


def run_accept(m, tree, logits, tokens, temperature, eps=0.09, delta=0.3):
    import torch
    B, T, V = logits.shape
    lg = dev(logits)
    tk = dev(np.asarray(tokens, np.int32))
    ws = m.workspace(m.typical_accept_workspace(B, T, V, tree.dims["n_internal"]))
    best = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    alen = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    m.typical_accept(lg, tk, tree, temperature, eps, delta, best, alen, ws, next_token=nxt)
    torch.cuda.synchronize()
    return host(best), host(alen), host(nxt)


def _tree_and_tokens(m, choices, K, topk, B, V, seed):
    import torch
    st = oracle.build_static(choices, topk, K)
    tree = m.Tree(choices, K, topk)
    rng = rng_for(seed, 11)
    topk_ids = np.stack([np.stack([rng.choice(V, size=topk, replace=False) for _ in range(K)])
                         for _ in range(B)]).astype(np.int32)
    root = rng.integers(0, V, B).astype(np.int32)
    tokens, _ = oracle.gather(st, topk_ids, root, [0] * B)
    T = st["T"]
    tt = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    pp = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    m.build_tree(tree, dev(topk_ids), dev(root), dev(np.zeros(B, np.int32)), tt, pp)
    return st, tree, np.array(tokens, np.int32)


def _compare(st, res, logits, dtype, got):
    cands, nband = accept_candidates(st, res, logits, dtype)
    best, alen, nxt = got
    for b in range(len(cands)):
        assert (int(best[b]), int(alen[b]), int(nxt[b])) in cands[b], (b, best[b], alen[b], nxt[b], cands[b])
    return nband


@pytest.mark.parametrize("ci,temp", [(0, 0.7), (1, 0.0), (1, 0.7), (2, 0.0), (2, 0.7), (3, 0.7),
                                     (4, 0.0), (4, 0.7)])
def test_accept_full_size(ci, temp):
    cfg = get_config(ci)
    m = lib()
    st, tree, tokens = _tree_and_tokens(m, load_tree_choices(f"c{ci}"), cfg.K, cfg.topk, cfg.B,
                                        cfg.V, seed=ci)
    logits = gen_verif_logits(cfg, st["parent"], tokens)
    t32 = float(np.float32(temp))
    res = oracle.typical_accept(logits, cfg.dtype, tokens, st, t32, float(np.float32(0.09)),
                                float(np.float32(0.3)))
    say("accept full size", cfg.name, temp)
    got = run_accept(m, tree, logits, tokens, temp)
    nband = _compare(st, res, logits, cfg.dtype, got)
    print(f"{cfg.name} T={temp}: accept_length {got[1].tolist()} oracle {res['accept_length'].tolist()}"
          f" banded {nband}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,tree,B,temp", [
    (1, "one", 1, 0.7), (7, "c0", 2, 0.7), (2047, "c1", 3, 1.0), (2049, "c1", 3, 0.0),
    (5000, "chain6", 2, 0.7), (4100, "c3", 5, 0.3), (300, "c2", 8, 3.0),
    (20001, "c4", 5, 0.7),      # 555 rows: 2 rounds per chunk, element loads (V % 8 != 0)
    (131072, "chain8", 16, 0.7),   # 128 rows: 4 rounds per chunk, vector loads
    (131077, "chain8", 16, 0.0),   # 4 rounds per chunk, element loads, ragged last chunk
    (1000, "max4096", 2, 0.7),     # the largest tree: 4096 tokens, 64 internal rows, 4032 paths
    (1000, "max4096", 2, 0.0),
])
def test_accept_edges(dtype, V, tree, B, temp):
    m = lib()
    if tree == "one":
        choices, K, topk = [[0]], 1, 1
    elif tree == "max4096":
        choices, K, topk = cartesian_choices([63, 64]), 2, 64
    elif tree in ("chain6", "chain8"):
        depth = int(tree[5:])
        choices, K, topk = cartesian_choices([1] * depth), depth, 1
    else:
        choices, K, topk = load_tree_choices(tree), 5, 10
    topk = min(topk, V)
    choices = [c for c in choices if max(c) < topk]
    st, tr, tokens = _tree_and_tokens(m, choices, K, topk, B, V, seed=V + B)
    cfg = custom(dtype=dtype, B=B, V=V, seed=V * 3 + B, boost_p=0.8)
    logits = gen_verif_logits(cfg, st["parent"], tokens)
    t32 = float(np.float32(temp))
    res = oracle.typical_accept(logits, dtype, tokens, st, t32, float(np.float32(0.09)),
                                float(np.float32(0.3)))
    say("accept edge", dtype, V, tree, B, temp)
    _compare(st, res, logits, dtype, run_accept(m, tr, logits, tokens, temp))


def test_accept_uniform_rows_accept_everything_and_neg_inf_rows():
    m = lib()
    choices = load_tree_choices("c1")
    V, B = 3000, 2
    st, tr, tokens = _tree_and_tokens(m, choices, 4, 10, B, V, seed=1)
    logits = np.zeros((B, st["T"], V), np.float32)            # b = 0: uniform -> all accepted
    logits[1] = -np.inf                                        # b = 1: one finite entry per row
    for n in range(st["T"]):
        logits[1, n, 17] = 1.0
    say("accept uniform / -inf rows")
    best, alen, nxt = run_accept(m, tr, logits, tokens, 0.7)
    res = oracle.typical_accept(logits, "f32", tokens, st, 0.7)
    assert alen[0] == max(st["path_len"]) == res["accept_length"][0]
    assert best[0] == res["best_candidate"][0] and nxt[0] == 0
    assert (best[1], alen[1], nxt[1]) == (res["best_candidate"][1], res["accept_length"][1], 17)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_accept_signed_zero_maxima_tie(dtype):
    """A row whose maximum is 0, held as -0 at index 2, +0 at 6 and -0 at 9 (2 and 6 in one
    thread's eight elements, 9 in the next): the zeros compare equal, so the argmax is the
    first of them, 2, as the oracle's numeric argmax has it.  Greedy: no candidate token is 2,
    so nothing is accepted and the next token is the root row's argmax."""
    m = lib()
    choices = load_tree_choices("c1")
    V, B = 3000, 1
    st, tr, tokens = _tree_and_tokens(m, choices, 4, 10, B, V, seed=2)
    tokens = np.where(tokens == 2, 3, tokens).astype(np.int32)
    f = np.full((B, st["T"], V), -1.0, np.float32)
    f[:, :, [2, 9]] = -0.0
    f[:, :, 6] = 0.0
    logits = f if dtype == "f32" else (f.view(np.uint32) >> 16).astype(np.uint16)
    say("accept signed zeros", dtype)
    best, alen, nxt = run_accept(m, tr, logits, tokens, 0.0)
    res = oracle.typical_accept(logits, dtype, tokens, st, 0.0)
    assert res["accept_length"][0] == 0 and res["next_token"][0] == 2
    assert (int(alen[0]), int(nxt[0])) == (0, 2)


def test_accept_strict_parameters_and_determinism():
    m = lib()
    cfg = get_config(1)
    st, tr, tokens = _tree_and_tokens(m, load_tree_choices("c1"), 4, 10, 1, cfg.V, seed=5)
    logits = gen_verif_logits(cfg, st["parent"], tokens, seed=55)
    res = oracle.typical_accept(logits, "bf16", tokens, st, float(np.float32(0.7)),
                                float(np.float32(0.12)), float(np.float32(0.35)))
    say("accept strict params")
    got = run_accept(m, tr, logits, tokens, 0.7, 0.12, 0.35)
    _compare(st, res, logits, "bf16", got)
    got2 = run_accept(m, tr, logits, tokens, 0.7, 0.12, 0.35)
    assert all(np.array_equal(x, y) for x, y in zip(got, got2))


SWEEP = [(0, 0.7, 16), (1, 0.0, 16), (1, 0.7, 16), (2, 0.0, 16), (2, 0.7, 16), (3, 0.7, 4),
         (4, 0.0, 4), (4, 0.7, 4)]


@pytest.mark.parametrize("ci,temp,nseeds", SWEEP)
def test_accept_seed_sweep(ci, temp, nseeds):
    """Every workload shape over several seeds (16 on the three smaller, 4 on the two largest):
    fresh tree tokens and verification logits per seed.  Decisions inside the 1e-4 band may go
    either way; their number is bounded (at most 1 in 500 of the decisions, and at least 2)."""
    cfg = get_config(ci)
    m = lib()
    choices = load_tree_choices(f"c{ci}")
    banded = decisions = 0
    lens = []
    for j in range(nseeds):
        seed = 100 + j
        st, tree, tokens = _tree_and_tokens(m, choices, cfg.K, cfg.topk, cfg.B, cfg.V, seed=seed)
        logits = gen_verif_logits(cfg, st["parent"], tokens, seed=seed)
        res = oracle.typical_accept(logits, cfg.dtype, tokens, st, float(np.float32(temp)),
                                    float(np.float32(0.09)), float(np.float32(0.3)))
        say("accept seed sweep", cfg.name, temp, seed)
        got = run_accept(m, tree, logits, tokens, temp)
        banded += _compare(st, res, logits, cfg.dtype, got)
        decisions += cfg.B * (st["T"] - 1)
        lens += got[1].tolist()
    print(f"{cfg.name} T={temp}: {nseeds} seeds, accept lengths {lens}, "
          f"banded {banded} of {decisions} decisions")
    assert banded <= max(2, decisions // 500)
