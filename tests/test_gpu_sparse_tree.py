"""The sparse candidate tree on the device path: the library's medusa_sparse_tree choice list goes
through build_tree, tree_attention and typical_accept on the GPU, against the oracle's
sparse_tree -> build_static -> gather -> tree attention -> typical acceptance (Ultralytics
"Medusa Heads", tree-attention section: a sparse tree of the most accurate candidate
combinations is what the step verifies)."""

import numpy as np
import pytest

import oracle
import oracle.sparse_tree as ost
from gpu_util import accept_candidates, as_f64, dev, host, lib, mask_array, say, tol
from synth import gen_attention_inputs, gen_verif_logits
from synth.configs import custom
from synth.gen import rng_for

pytestmark = pytest.mark.gpu


def _accuracy(kind, K, topk, seed):
    if kind == "model":          # top-1 0.60, top-5 > 0.80 per head (Wiblog, heads section)
        return np.array([[0.6 * (r + 1) ** -2.35 for r in range(topk)]] * K)
    rng = rng_for(seed, 31)
    a = rng.random((K, topk))
    return a / a.sum(1, keepdims=True) * rng.uniform(0.5, 0.95, (K, 1))


@pytest.mark.parametrize("kind,K,N,dtype,B,Hq,Hkv,L,V,temp", [
    ("model", 4, 64, "bf16", 1, 32, 32, 1024, 32000, 0.7),     # the 7B-shaped step
    ("model", 5, 64, "bf16", 1, 32, 8, 4096, 128256, 0.0),     # the Llama-8B-shaped step
    ("random", 3, 128, "bf16", 2, 16, 16, 777, 32000, 0.7),
    ("random", 2, 30, "f32", 3, 4, 2, 100, 1000, 1.0),
])
def test_sparse_tree_through_the_step(kind, K, N, dtype, B, Hq, Hkv, L, V, temp):
    import torch
    m = lib()
    topk = 10
    acc = _accuracy(kind, K, topk, seed=K * 1000 + N)
    choices, e = m.sparse_tree(acc, N)
    ref_choices, e_ref = ost.sparse_tree(acc.tolist(), N)
    assert choices == ref_choices and e == e_ref
    st = oracle.build_static(ref_choices, topk, K)
    T = st["T"]
    cfg = custom(dtype=dtype, B=B, V=V, K=K, topk=topk, Hq=Hq, Hkv=Hkv, D=128 if dtype == "bf16" else 64,
                 L=L, seed=N + K, boost_p=0.7)
    rng = rng_for(cfg.seed, 12)
    ids = np.stack([np.stack([rng.choice(V, size=topk, replace=False) for _ in range(K)])
                    for _ in range(B)]).astype(np.int32)
    root = rng.integers(0, V, B).astype(np.int32)
    pl = np.full(B, L, np.int32)
    tokens, pos = oracle.gather(st, ids, root, pl)
    a = gen_attention_inputs(cfg, T)
    att = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], dtype, pl, st["mask"], Hkv)
    logits = gen_verif_logits(cfg, st["parent"], np.array(tokens))
    res = oracle.typical_accept(logits, dtype, tokens, st, float(np.float32(temp)),
                                float(np.float32(0.09)), float(np.float32(0.3)))

    say("sparse tree step", kind, K, N, dtype, B, Hq, Hkv, L, V, temp)
    tree = m.Tree(choices, K, topk)
    tt = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    pp = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    m.build_tree(tree, dev(ids), dev(root), dev(pl), tt, pp)
    q = dev(a["q"])
    out = torch.full_like(q, float("nan"))
    ws = m.workspace(m.tree_attention_workspace(B, Hq, Hkv, T, cfg.D, L))
    m.tree_attention(q, dev(a["k_cache"]), dev(a["v_cache"]), dev(pl), L, tree.mask, out, ws)
    best = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    alen = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    wa = m.workspace(m.typical_accept_workspace(B, T, V, tree.dims["n_internal"]))
    m.typical_accept(dev(logits), tt, tree, temp, 0.09, 0.3, best, alen, wa, next_token=nxt)
    torch.cuda.synchronize()

    assert np.array_equal(host(tree.mask).view(np.uint64), mask_array(st))
    assert host(tt).tolist() == tokens and host(pp).tolist() == pos
    err = float(np.abs(as_f64(host(out), dtype) - att).max())
    assert err <= tol(dtype), err
    cands, nband = accept_candidates(st, res, logits, dtype)
    got = (host(best), host(alen), host(nxt))
    for b in range(B):
        assert (int(got[0][b]), int(got[1][b]), int(got[2][b])) in cands[b]
    print(f"{kind} K={K} N={N}: E[accept length] {e:.4f}, attention err {err:.2e}, "
          f"accept_length {got[1].tolist()} banded {nband}")
