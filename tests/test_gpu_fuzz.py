"""Randomised small steps on the GPU against the oracle: random prefix-closed trees (up to 40
tokens, depth up to 6), vocab sizes around the 64-element boundaries, hidden sizes 8 / 64 / 264,
prefixes of 0, 1, 127 and 129 tokens, query groups of 1, 2 and 8, both dtypes, three
temperatures, both acceptance modes; then plain causal attention over [prefix; path] for every
root-to-leaf path against the tree attention output of each node on it (Wiblog page,
tree-attention section: a token sees only its own path)."""

import numpy as np
import pytest

import oracle
from gpu_util import accept_candidates, as_f64, check_topk, dev, host, lib, say, tol
from synth.configs import custom
from synth.gen import gen_attention_inputs, gen_head_inputs, gen_verif_logits, rng_for

pytestmark = pytest.mark.gpu

N_CASES = 64


def random_tree(rng, max_tokens=40, max_depth=6, topk=8):
    """A random prefix-closed choice list: nodes are added under random existing nodes, each new
    child taking its parent's next free rank (so every rank is < topk)."""
    nodes = [()]
    used = {(): 0}
    target = int(rng.integers(1, max_tokens))
    while len(nodes) < target + 1:
        parent = nodes[int(rng.integers(len(nodes)))]
        if len(parent) >= max_depth or used[parent] >= topk:
            if all(len(p) >= max_depth or used[p] >= topk for p in nodes):
                break
            continue
        child = parent + (used[parent],)
        used[parent] += 1
        used[child] = 0
        nodes.append(child)
    return [list(t) for t in nodes[1:]]


def _case(i):
    rng = rng_for(900 + i, 0)
    V = int(rng.choice([1, 63, 64, 65, 257, 1000]))
    topk = int(min(V, rng.integers(1, 9)))
    choices = random_tree(rng, topk=topk)
    depth = max(len(c) for c in choices)
    K = int(rng.integers(depth, 7))
    dtype = "bf16" if i % 2 else "f32"
    Hd = int(rng.choice([8, 64, 264]))
    G = int(rng.choice([1, 2, 8]))
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    pls = [int(x) for x in rng.choice([0, 1, 127, 129], size=B)]
    temp = float(rng.choice([0.0, 0.7, 1.3]))
    sampling = "nucleus" if rng.random() < 0.3 and temp > 0 else "typical"
    top_p = float(rng.uniform(0.2, 1.0))
    packed = dtype == "bf16" and Hd % 32 == 0 and rng.random() < 0.5
    return dict(V=V, topk=topk, choices=choices, K=K, dtype=dtype, Hd=Hd, G=G, Hkv=Hkv, B=B, D=D,
                pls=pls, temp=temp, sampling=sampling, top_p=top_p, packed=packed, seed=900 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_step(i):
    import torch
    c = _case(i)
    m = lib()
    cfg = custom(dtype=c["dtype"], B=c["B"], Hd=c["Hd"], V=c["V"], K=c["K"], topk=c["topk"],
                 Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"], L=max(c["pls"]),
                 w_std=1.0 / np.sqrt(c["Hd"]), seed=c["seed"], boost_p=0.7)
    say("fuzz", i, {k: v for k, v in c.items() if k != "choices"}, "T", len(c["choices"]) + 1)
    # ---- oracle chain ----
    hin = gen_head_inputs(cfg)
    _, l64 = oracle.heads(hin["h"], hin["w1"], hin["b1"], hin["w2"], cfg.dtype)
    ids64, _ = oracle.topk(l64, cfg.topk)
    ties = oracle.topk_ties(l64, cfg.topk)
    st = oracle.build_static(c["choices"], cfg.topk, cfg.K)
    T = st["T"]
    root = rng_for(c["seed"], 4).integers(0, cfg.V, cfg.B).astype(np.int32)
    pl = np.asarray(c["pls"], np.int32)
    tokens, pos = oracle.gather(st, ids64, root, pl)
    a = gen_attention_inputs(cfg, T, prefix_lens=pl)
    att = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, pl, st["mask"],
                                cfg.Hkv)
    logits = gen_verif_logits(cfg, st["parent"], np.array(tokens))
    # ---- GPU chain ----
    step = m.VerifyStep(B=cfg.B, hidden=cfg.Hd, vocab=cfg.V, K=cfg.K, topk=cfg.topk,
                        choices=c["choices"], Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D,
                        max_prefix_len=int(pl.max()))
    w1, w2 = dev(hin["w1"]), dev(hin["w2"])
    if c["packed"]:
        w1, w2 = m.pack_weights(w1), m.pack_weights(w2)
    q = dev(a["q"])
    out = torch.full_like(q, float("nan"))
    step.heads_and_tree(dev(hin["h"]), w1, dev(hin["b1"]), w2, dev(root), dev(pl))
    step.attention(q, dev(a["k_cache"]), dev(a["v_cache"]), dev(pl), out)
    best = torch.full((cfg.B,), -1, dtype=torch.int32, device="cuda")
    alen = torch.full((cfg.B,), -1, dtype=torch.int32, device="cuda")
    nxt = torch.full((cfg.B,), -1, dtype=torch.int32, device="cuda")
    ws = m.workspace(m.evaluate_posterior_workspace(cfg.B, cfg.V, step.tree, c["sampling"]))
    m.evaluate_posterior(dev(logits), step.tokens, step.tree, c["temp"], 0.09, 0.3, best, alen, ws,
                         top_p=c["top_p"], sampling=c["sampling"], next_token=nxt)
    torch.cuda.synchronize()
    # ---- compare ----
    assert float(np.abs(host(step.logits) - l64).max()) <= tol(cfg.dtype)
    check_topk(host(step.topk_ids), l64, cfg.topk)
    tk = host(step.tokens)
    for b in range(cfg.B):
        for n, t in enumerate(st["nodes"]):
            if len(t) == 0 or not ties[b, len(t) - 1]:
                assert tk[b, n] == tokens[b][n], (b, n)
    assert host(step.position_ids).tolist() == pos
    got = as_f64(host(out), cfg.dtype)
    assert not np.isnan(got).any()
    assert float(np.abs(got - att).max()) <= tol(cfg.dtype)
    res = oracle.evaluate_posterior(logits, cfg.dtype, tokens, st, float(np.float32(c["temp"])),
                                    float(np.float32(0.09)), float(np.float32(0.3)),
                                    top_p=float(np.float32(c["top_p"])), sampling=c["sampling"])
    cands, _ = accept_candidates(st, res, logits, cfg.dtype)
    for b in range(cfg.B):
        assert (int(host(best)[b]), int(host(alen)[b]), int(host(nxt)[b])) in cands[b]
    # ---- every root-to-leaf path as plain causal attention over [prefix; path] ----
    scale = 1.0 / np.sqrt(cfg.D)
    kc, vc = as_f64(a["k_cache"], cfg.dtype), as_f64(a["v_cache"], cfg.dtype)
    qq = as_f64(a["q"], cfg.dtype)
    for b in range(cfg.B):
        L = int(pl[b])
        for path, plen in zip(st["paths"], st["path_len"]):
            nodes = path[:plen + 1]
            for hq in range(cfg.Hq):
                g = hq // c["G"]
                keys = np.concatenate([kc[b, g, :L], kc[b, g, [L + n for n in nodes]]])
                vals = np.concatenate([vc[b, g, :L], vc[b, g, [L + n for n in nodes]]])
                for t, n in enumerate(nodes):
                    s = keys[:L + t + 1] @ qq[b, hq, n] * scale
                    w = np.exp(s - s.max())
                    ref = (w[:, None] * vals[:L + t + 1]).sum(0) / w.sum()
                    assert float(np.abs(got[b, hq, n] - ref).max()) <= tol(cfg.dtype)
