"""GPU parity of commit_accepted against the oracle, through the C ABI: bit-exact (it moves data
and integers only).  Whole caches are compared, so a stray write anywhere fails."""

import numpy as np
import pytest

import oracle
from gpu_util import dev, host, lib, say
from synth import get_config
from synth.configs import custom
from synth.gen import gen_attention_inputs, rng_for
from synth.trees import cartesian_choices, load_tree_choices

pytestmark = pytest.mark.gpu


def _case(m, choices, topk, K, cfg, pls, seed, lcap_extra=5, hidden_size=64):
    import torch
    st = oracle.build_static(choices, topk, K)
    tree = m.Tree(choices, K, topk)
    T = st["T"]
    B = cfg.B
    z = torch.zeros(B, dtype=torch.int32, device="cuda")
    tt = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    m.build_tree(tree, torch.zeros((B, K, topk), dtype=torch.int32, device="cuda"), z, z, tt,
                 torch.zeros_like(tt))                   # uploads the static tree arrays
    a = gen_attention_inputs(cfg, T, prefix_lens=pls, lcap=max(pls) + T + lcap_extra)
    rng = rng_for(seed, 13)
    tokens = rng.integers(0, 50000, (B, T)).astype(np.int32)
    P = len(st["paths"])
    best = rng.integers(0, P, B).astype(np.int32)
    alen = np.array([rng.integers(0, st["path_len"][p] + 1) for p in best], np.int32)
    nxt = rng.integers(0, 50000, B).astype(np.int32)
    hdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    hidden = (rng.integers(0, 65535, (B, T, hidden_size)).astype(np.uint16) if cfg.dtype == "bf16"
              else rng.standard_normal((B, T, hidden_size)).astype(np.float32)).astype(hdt)
    return st, tree, a, tokens, best, alen, nxt, hidden


def _run(m, st, tree, a, tokens, best, alen, nxt, hidden, alias=False):
    import torch
    B = len(best)
    kc, vc = dev(a["k_cache"]), dev(a["v_cache"])
    pl = dev(a["prefix_len"])
    npl = pl if alias else torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out_tokens = torch.full((B, st["dmax"] + 1), -9, dtype=torch.int32, device="cuda")
    out_count = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    root = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    hd = dev(hidden)
    nh = torch.zeros((B, hidden.shape[2]), dtype=hd.dtype, device="cuda")
    m.commit_accepted(tree, dev(best), dev(alen), dev(tokens), dev(nxt), kc, vc, pl, npl,
                      out_tokens, out_count, new_root=root, hidden=hd, next_hidden=nh)
    torch.cuda.synchronize()
    return dict(k_cache=host(kc), v_cache=host(vc), prefix_len=host(npl),
                out_tokens=host(out_tokens), out_count=host(out_count), new_root=host(root),
                next_hidden=host(nh))


def _compare(got, ref):
    for k in ("k_cache", "v_cache", "prefix_len", "out_tokens", "out_count", "new_root",
              "next_hidden"):
        g, r = np.asarray(got[k]), np.asarray(ref[k])
        assert np.array_equal(g, r), (k, g.ravel()[:8], r.ravel()[:8], got["out_count"], ref["out_count"])


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_commit_full_size(ci):
    cfg = get_config(ci)
    m = lib()
    st, tree, a, tokens, best, alen, nxt, hidden = _case(
        m, load_tree_choices(f"c{ci}"), cfg.topk, cfg.K, cfg, [cfg.L] * cfg.B, seed=ci + 40,
        hidden_size=cfg.Hd)
    say("commit full size", cfg.name, best.tolist(), alen.tolist())
    got = _run(m, st, tree, a, tokens, best, alen, nxt, hidden)
    ref = oracle.commit(st, best, alen, tokens, nxt, a["k_cache"], a["v_cache"], a["prefix_len"],
                        hidden)
    _compare(got, ref)


@pytest.mark.parametrize("dtype,D,tree,pls,alias", [
    ("bf16", 128, "c1", [0, 5, 300], False), ("bf16", 64, "c3", [17, 0], True),
    ("f32", 64, "c0", [3, 9, 1], False), ("f32", 128, "chain6", [40], True),
])
def test_commit_edges(dtype, D, tree, pls, alias):
    m = lib()
    if tree == "chain6":
        choices, topk, K = cartesian_choices([1] * 6), 1, 6
    else:
        choices, topk, K = load_tree_choices(tree), 10, 5
    cfg = custom(dtype=dtype, B=len(pls), Hq=4, Hkv=3, D=D, L=max(pls), seed=len(pls) + D)
    st, tr, a, tokens, best, alen, nxt, hidden = _case(m, choices, topk, K, cfg, pls, seed=D + 1,
                                                       hidden_size=96)
    alen[0] = 0                                                  # root only: nothing moves
    if len(pls) > 1:
        alen[-1] = st["path_len"][best[-1]]                      # a whole path
    say("commit edge", dtype, D, tree, pls, alias)
    got = _run(m, st, tr, a, tokens, best, alen, nxt, hidden, alias=alias)
    ref = oracle.commit(st, best, alen, tokens, nxt, a["k_cache"], a["v_cache"], a["prefix_len"],
                        hidden)
    _compare(got, ref)


def test_commit_out_of_range_inputs_leave_the_sequence_untouched():
    m = lib()
    cfg = custom(dtype="bf16", B=4, Hq=2, Hkv=2, D=64, L=8, seed=5)
    choices = load_tree_choices("c1")
    st, tree, a, tokens, best, alen, nxt, hidden = _case(m, choices, 10, 5, cfg, [8, 8, 8, 8],
                                                         seed=6, lcap_extra=0)
    P = len(st["paths"])
    best[1] = P                                   # no such path
    alen[2] = st["path_len"][best[2]] + 1         # longer than its path
    a["prefix_len"][3] = 9                        # L + T > lcap
    say("commit out of range")
    got = _run(m, st, tree, a, tokens, best, alen, nxt, hidden)
    ok = [0]
    ref = oracle.commit(st, best[ok], alen[ok], tokens[ok], nxt[ok], a["k_cache"][ok],
                        a["v_cache"][ok], a["prefix_len"][ok], hidden[ok])
    assert np.array_equal(got["k_cache"][0], ref["k_cache"][0])
    for b in (1, 2, 3):
        assert got["out_count"][b] == 0 and got["prefix_len"][b] == a["prefix_len"][b]
        assert (got["out_tokens"][b] == -1).all()
        assert np.array_equal(got["k_cache"][b], a["k_cache"][b])
        assert np.array_equal(got["v_cache"][b], a["v_cache"][b])
