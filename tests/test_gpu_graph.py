"""A step recorded into a HIP graph (VerifyStep.capture) and replayed: every replay, with eager
steps and new input contents in between, gives bit for bit the outputs of the eager step on the
same inputs (the graph holds kernel nodes only: nothing in the step clears or copies memory)."""

import numpy as np
import pytest

from gpu_util import dev, host, lib, say
from synth import (gen_attention_inputs, gen_head_inputs, gen_root_tokens, gen_verif_logits,
                   get_config, load_tree_choices)
from synth.gen import normals, rng_for

pytestmark = pytest.mark.gpu


def _outputs(step, out):
    return [host(t).copy() for t in (step.logits, step.topk_ids, step.tokens, step.position_ids,
                                      out, step.best, step.accept_length, step.next_token)]


@pytest.mark.parametrize("ci,packed", [(0, False), (1, True), (3, True)])
def test_graph_replay_matches_eager(ci, packed):
    import torch
    cfg = get_config(ci)
    m = lib()
    choices = load_tree_choices(f"c{ci}")
    hin = gen_head_inputs(cfg)
    step = m.VerifyStep(B=cfg.B, hidden=cfg.Hd, vocab=cfg.V, K=cfg.K, topk=cfg.topk,
                        choices=choices, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, max_prefix_len=cfg.L)
    T = step.tree.T
    w1, w2 = dev(hin["w1"]), dev(hin["w2"])
    if packed:
        w1, w2 = m.pack_weights(w1), m.pack_weights(w2)
    h, b1 = dev(hin["h"]), dev(hin["b1"])
    a = gen_attention_inputs(cfg, T)
    q, kc, vc = dev(a["q"]), dev(a["k_cache"]), dev(a["v_cache"])
    pl, root = dev(a["prefix_len"]), dev(gen_root_tokens(cfg))
    out = torch.zeros_like(q)
    # verification logits for a synthetic tree-token draw (their contents only need to be fixed)
    rng = rng_for(cfg.seed, 21)
    toks = rng.integers(0, cfg.V, (cfg.B, T)).astype(np.int32)
    parent = np.array([-1] + [0] * (T - 1))
    logits = dev(gen_verif_logits(cfg, parent, toks))
    temp = cfg.temps[-1]
    kw = dict(h=h, w1=w1, b1=b1, w2=w2, root_tokens=root, prefix_len=pl, q=q, k_cache=kc,
              v_cache=vc, attn_out=out, verif_logits=logits, temperature=temp,
              eps=cfg.eps, delta=cfg.delta)
    say("graph", cfg.name, "packed" if packed else "unpacked")
    step.run(**kw)
    torch.cuda.synchronize()
    eager = _outputs(step, out)
    graph = step.capture(**kw)
    for r in range(3):
        if r == 2:
            # new contents in the same buffers: another hidden state and other roots
            h.copy_(dev(normals((cfg.B, cfg.Hd), cfg.seed + 7, 0, 0, 1.0, cfg.dtype)))
            root.copy_((root.flip(0) + 1) % cfg.V)
            step.run(**kw)
            torch.cuda.synchronize()
            eager = _outputs(step, out)
        for t in (step.logits, step.topk_ids, step.tokens, out, step.best, step.accept_length):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(step, out)
        for i, (x, y) in enumerate(zip(got, eager)):
            assert np.array_equal(x, y), (r, i)
        step.run(**kw)          # eager work between replays
        torch.cuda.synchronize()
        assert all(np.array_equal(x, y) for x, y in zip(_outputs(step, out), eager))
    print(f"{cfg.name}: 3 replays equal to eager, accept_length {eager[6].tolist()}")
