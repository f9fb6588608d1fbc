"""End-to-end: the chained GPU step (VerifyStep: heads -> build_tree -> tree_attention ->
typical_accept, then the commit) against the chained oracle step, on the workloads' full shapes
and on the packed weights the benchmark times.  Attention outputs of the two largest workloads are
compared at sampled (sequence, head, node) units; everything else everywhere."""

import numpy as np
import pytest

import oracle
from gpu_util import (accept_candidates, as_f64, check_topk, dev, host, lib, sample_units, say,
                      tol)
from synth import (gen_attention_inputs, gen_head_inputs, gen_root_tokens, gen_verif_logits,
                   get_config, load_tree_choices)
from synth.configs import custom

pytestmark = pytest.mark.gpu


def _chain(m, cfg, choices, packed, prefix_len, full_attention):
    import torch
    # ---- oracle chain ----
    hin = gen_head_inputs(cfg)
    _, l64 = oracle.heads(hin["h"], hin["w1"], hin["b1"], hin["w2"], cfg.dtype)
    ids64, _ = oracle.topk(l64, cfg.topk)
    ties = oracle.topk_ties(l64, cfg.topk)
    st = oracle.build_static(choices, cfg.topk, cfg.K)
    T = st["T"]
    root = gen_root_tokens(cfg)
    pl = np.asarray(prefix_len, np.int32)
    tokens, pos = oracle.gather(st, ids64, root, pl)
    a = gen_attention_inputs(cfg, T, prefix_lens=pl)
    sel = None if full_attention else sample_units(cfg.B, cfg.Hq, T, 300, cfg.seed)
    att = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, pl, st["mask"],
                                cfg.Hkv, sel=sel)
    logits = gen_verif_logits(cfg, st["parent"], np.array(tokens))
    # ---- GPU chain ----
    step = m.VerifyStep(B=cfg.B, hidden=cfg.Hd, vocab=cfg.V, K=cfg.K, topk=cfg.topk,
                        choices=choices, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D,
                        max_prefix_len=int(pl.max()))
    w1, w2 = dev(hin["w1"]), dev(hin["w2"])
    if packed:
        w1, w2 = m.pack_weights(w1), m.pack_weights(w2)
    h, b1 = dev(hin["h"]), dev(hin["b1"])
    del hin
    q, kc, vc = dev(a["q"]), dev(a["k_cache"]), dev(a["v_cache"])
    out = torch.full_like(q, float("nan"))
    dlog, dpl, droot = dev(logits), dev(pl), dev(root)
    for temp in cfg.temps:
        say("step", cfg.name, "packed" if packed else "unpacked", temp, "prefix", pl.tolist())
        step.run(h=h, w1=w1, b1=b1, w2=w2, root_tokens=droot, prefix_len=dpl, q=q, k_cache=kc,
                 v_cache=vc, attn_out=out, verif_logits=dlog, temperature=temp)
        torch.cuda.synchronize()
        lerr = float(np.abs(host(step.logits) - l64).max())
        assert lerr <= tol(cfg.dtype), lerr
        check_topk(host(step.topk_ids), l64, cfg.topk)
        if ties.any():      # a tied top-k row may legitimately order its ids otherwise
            print(f"{cfg.name}: {int(ties.sum())} top-k tie rows; tokens compared outside them")
        tk = host(step.tokens)
        for b in range(cfg.B):
            for i, t in enumerate(st["nodes"]):
                if len(t) == 0 or not ties[b, len(t) - 1]:
                    assert tk[b, i] == tokens[b][i], (b, i)
        assert host(step.position_ids).tolist() == pos
        got_att = as_f64(host(out), cfg.dtype)
        if sel is None:
            assert not np.isnan(got_att).any()
            aerr = float(np.abs(got_att - att).max())
        else:
            aerr = float(np.abs(got_att[sel[:, 0], sel[:, 1], sel[:, 2]]
                                - att[sel[:, 0], sel[:, 1], sel[:, 2]]).max())
        assert aerr <= tol(cfg.dtype), aerr
        res = oracle.typical_accept(logits, cfg.dtype, tokens, st, float(np.float32(temp)),
                                    float(np.float32(cfg.eps)), float(np.float32(cfg.delta)))
        cands, nband = accept_candidates(st, res, logits, cfg.dtype)
        got = (host(step.best), host(step.accept_length), host(step.next_token))
        for b in range(cfg.B):
            assert (int(got[0][b]), int(got[1][b]), int(got[2][b])) in cands[b]
        print(f"{cfg.name} T={temp}: logits err {lerr:.2e}, attention err {aerr:.2e}, "
              f"best {got[0].tolist()} accept_length {got[1].tolist()} banded {nband}")
        # ---- commit the accepted candidate (on copies of the caches) against the oracle ----
        kc2, vc2 = kc.clone(), vc.clone()
        hid = np.arange(cfg.B * T * 16, dtype=np.float32).reshape(cfg.B, T, 16)
        hid = hid.view(np.uint32).astype(np.uint16) if cfg.dtype == "bf16" else hid
        nh = torch.zeros((cfg.B, 16), dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                         device="cuda")
        step.commit(kc2, vc2, dpl, hidden=dev(hid), next_hidden=nh)
        torch.cuda.synchronize()
        ref = oracle.commit(st, got[0], got[1], host(step.tokens).tolist(), got[2], a["k_cache"],
                            a["v_cache"], pl, hid)
        assert np.array_equal(host(kc2), ref["k_cache"]) and np.array_equal(host(vc2), ref["v_cache"])
        assert np.array_equal(host(step.out_tokens), ref["out_tokens"])
        assert np.array_equal(host(step.out_count), ref["out_count"])
        assert np.array_equal(host(step.new_prefix_len), ref["prefix_len"])
        assert np.array_equal(host(step.new_root), ref["new_root"])
        assert np.array_equal(host(nh), ref["next_hidden"])
        del kc2, vc2


@pytest.mark.parametrize("ci,packed", [(0, False), (1, False), (1, True), (2, True), (3, True),
                                       (4, True)])
def test_step_end_to_end(ci, packed):
    cfg = get_config(ci)
    _chain(lib(), cfg, load_tree_choices(f"c{ci}"), packed, [cfg.L] * cfg.B,
           full_attention=ci <= 2)


def test_step_ragged_prefixes_batch8_gqa():
    """Eight sequences with ragged prefixes (0 and 1 included) on the 128-node tree, grouped
    query heads, packed weights: the batch-8 vocab projection variant, the per-sequence prefix
    of attention and commit, and the batch paths of acceptance, chained."""
    cfg = custom(name="b8_ragged_bf16", dtype="bf16", B=8, Hd=1024, V=32000, K=3, topk=10, Hq=16,
                 Hkv=4, D=128, L=700, tree="c3", temps=(0.0, 0.7), boost_p=0.7, seed=38,
                 w_std=1.0 / np.sqrt(1024))
    _chain(lib(), cfg, load_tree_choices("c3"), True, [700, 1, 333, 0, 517, 64, 128, 699],
           full_attention=True)
