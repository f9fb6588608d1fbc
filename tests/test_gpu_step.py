"""End-to-end: the chained GPU step (VerifyStep) against the chained oracle step."""

import numpy as np
import pytest

import oracle
from gpu_util import accept_candidates, as_f64, check_topk, dev, host, lib, say, tol
from synth import (gen_attention_inputs, gen_head_inputs, gen_root_tokens, gen_verif_logits,
                   get_config, load_tree_choices)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ci", [0, 1])
def test_step_end_to_end(ci):
    import torch
    cfg = get_config(ci)
    m = lib()
    choices = load_tree_choices(f"c{ci}")
    # ---- oracle chain ----
    hin = gen_head_inputs(cfg)
    _, l64 = oracle.heads(hin["h"], hin["w1"], hin["b1"], hin["w2"], cfg.dtype)
    ids64, _ = oracle.topk(l64, cfg.topk)
    st = oracle.build_static(choices, cfg.topk, cfg.K)
    root = gen_root_tokens(cfg)
    pl = np.full(cfg.B, cfg.L, np.int32)
    tokens, pos = oracle.gather(st, ids64, root, pl)
    a = gen_attention_inputs(cfg, st["T"])
    att = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, pl, st["mask"], cfg.Hkv)
    logits = gen_verif_logits(cfg, st["parent"], np.array(tokens))
    # ---- GPU chain ----
    step = m.VerifyStep(B=cfg.B, hidden=cfg.Hd, vocab=cfg.V, K=cfg.K, topk=cfg.topk,
                        choices=choices, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, max_prefix_len=cfg.L)
    q, kc, vc = dev(a["q"]), dev(a["k_cache"]), dev(a["v_cache"])
    out = torch.empty_like(q)
    dlog = dev(logits)
    for temp in cfg.temps:
        say("step", cfg.name, temp)
        step.run(h=dev(hin["h"]), w1=dev(hin["w1"]), b1=dev(hin["b1"]), w2=dev(hin["w2"]),
                 root_tokens=dev(root), prefix_len=dev(pl), q=q, k_cache=kc, v_cache=vc,
                 attn_out=out, verif_logits=dlog, temperature=temp)
        torch.cuda.synchronize()
        check_topk(host(step.topk_ids), l64, cfg.topk)
        assert host(step.tokens).tolist() == tokens
        assert host(step.position_ids).tolist() == pos
        assert float(np.abs(as_f64(host(out), cfg.dtype) - att).max()) <= tol(cfg.dtype)
        res = oracle.typical_accept(logits, cfg.dtype, tokens, st, float(np.float32(temp)),
                                    float(np.float32(0.09)), float(np.float32(0.3)))
        cands, _ = accept_candidates(st, res, logits, cfg.dtype)
        got = (host(step.best), host(step.accept_length), host(step.next_token))
        for b in range(cfg.B):
            assert (int(got[0][b]), int(got[1][b]), int(got[2][b])) in cands[b]
        print(f"{cfg.name} T={temp}: best {got[0].tolist()} accept_length {got[1].tolist()}")
        # ---- commit the accepted candidate (on copies of the caches) against the oracle ----
        kc2, vc2 = kc.clone(), vc.clone()
        hid = np.arange(cfg.B * st["T"] * 16, dtype=np.float32).reshape(cfg.B, st["T"], 16)
        hid = hid.view(np.uint32).astype(np.uint16) if cfg.dtype == "bf16" else hid
        nh = torch.zeros((cfg.B, 16), dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                         device="cuda")
        step.commit(kc2, vc2, dev(pl), hidden=dev(hid), next_hidden=nh)
        torch.cuda.synchronize()
        ref = oracle.commit(st, got[0], got[1], tokens, got[2], a["k_cache"], a["v_cache"], pl, hid)
        assert np.array_equal(host(kc2), ref["k_cache"]) and np.array_equal(host(vc2), ref["v_cache"])
        assert np.array_equal(host(step.out_tokens), ref["out_tokens"])
        assert np.array_equal(host(step.out_count), ref["out_count"])
        assert np.array_equal(host(step.new_prefix_len), ref["prefix_len"])
        assert np.array_equal(host(step.new_root), ref["new_root"])
        assert np.array_equal(host(nh), ref["next_hidden"])

