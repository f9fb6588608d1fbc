"""GPU parity of medusa_heads_ex (heads of several residual blocks, optionally with LayerNorm)
against the oracle, through the C ABI: logits within the head tolerance, top-k ids exact (up to
ties).  One block without LayerNorm must equal medusa_heads bit for bit, and zero-initialised
blocks must leave h untouched, so their logits equal the single-block zero-init logits bit for
bit."""

import numpy as np
import pytest

import oracle
from gpu_util import check_topk, dev, host, lib, say, tol
from synth.gen import normals


def _inputs(dtype, B, hd, V, K, nb, ln, seed):
    std = 1.0 / np.sqrt(hd)
    h = normals((B, hd), seed, 20, 0, 1.0, dtype)
    w1 = normals((K, nb, hd, hd), seed, 20, 1, std, dtype)
    b1 = normals((K, nb, hd), seed, 20, 2, std, dtype)
    w2 = normals((K, V, hd), seed, 20, 3, std, dtype)
    g = normals((K, nb, hd), seed, 20, 4, 0.2, dtype) if ln else None
    be = normals((K, nb, hd), seed, 20, 5, 0.2, dtype) if ln else None
    if ln:                                       # gamma around 1
        g64 = oracle.head_blocks._f64(g, dtype) + 1.0
        g = (g64.astype(np.float32) if dtype == "f32" else
             (g64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    return h, w1, b1, w2, g, be


def _run(m, h, w1, b1, w2, g, be, dtype, packed, V, K, nb, topk):
    import torch
    B, hd = h.shape
    ws = m.workspace(m.medusa_heads_ex_workspace(B, hd, V, K, nb, g is not None, topk))
    logits = torch.full((B, K, V), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((B, K, topk), -1, dtype=torch.int32, device="cuda")
    dw1, dw2 = dev(w1), dev(w2)
    if packed:
        dw1 = m.pack_weights(dw1.reshape(K * nb, hd, hd))
        dw2 = m.pack_weights(dw2)
    m.medusa_heads_ex(dev(h), dw1, dev(b1), dw2, V, K, nb, topk, ids, ws,
                      ln_gamma=None if g is None else dev(g), ln_beta=None if be is None else dev(be),
                      packed=packed, logits=logits)
    torch.cuda.synchronize()
    return host(logits), host(ids)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,packed,nb,ln,B,hd,V,K", [
    ("f32", False, 2, False, 2, 256, 1000, 3),
    ("f32", False, 3, True, 1, 256, 777, 2),
    ("bf16", False, 2, True, 3, 512, 3000, 2),
    ("bf16", False, 2, True, 2, 264, 1000, 3),      # hidden a multiple of 8, not of 32
    ("f32", False, 2, True, 3, 8, 50, 2),
    ("bf16", True, 3, False, 1, 1024, 5000, 3),
    ("bf16", True, 2, True, 8, 512, 2000, 2),
    ("bf16", True, 2, True, 1, 4096, 32000, 4),     # the Vicuna-7B head shape with 2 LN blocks
])
def test_heads_ex_matches_oracle(dtype, packed, nb, ln, B, hd, V, K):
    m = lib()
    topk = 10
    h, w1, b1, w2, g, be = _inputs(dtype, B, hd, V, K, nb, ln, seed=hd + nb)
    say("heads_ex", dtype, packed, nb, ln, B, hd, V, K)
    lg, ids = _run(m, h, w1, b1, w2, g, be, dtype, packed, V, K, nb, topk)
    _, ref = oracle.heads_blocks(h, w1, b1, w2, dtype, g, be)
    err = float(np.abs(lg - ref).max())
    print(f"heads_ex {dtype} packed={packed} nb={nb} ln={ln}: max |logit - oracle| = {err:.3e}")
    assert err <= tol(dtype)
    check_topk(ids, ref, topk)


@pytest.mark.gpu
@pytest.mark.parametrize("packed", [False, True])
def test_one_block_is_medusa_heads(packed):
    import torch
    m = lib()
    B, hd, V, K, topk = 2, 512, 4000, 3, 10
    h, w1, b1, w2, _, _ = _inputs("bf16", B, hd, V, K, 1, False, seed=7)
    say("heads_ex one block", packed)
    lg, ids = _run(m, h, w1, b1, w2, None, None, "bf16", packed, V, K, 1, topk)
    ws = m.workspace(m.medusa_heads_workspace(B, hd, V, K, topk))
    ref = torch.full((B, K, V), float("nan"), dtype=torch.float32, device="cuda")
    rid = torch.full((B, K, topk), -1, dtype=torch.int32, device="cuda")
    if packed:
        m.medusa_heads_packed(dev(h), m.pack_weights(dev(w1[:, 0])), dev(b1[:, 0]),
                              m.pack_weights(dev(w2)), V, K, topk, rid, ws, logits=ref)
    else:
        m.medusa_heads(dev(h), dev(w1[:, 0]), dev(b1[:, 0]), dev(w2), topk, rid, ws, logits=ref)
    torch.cuda.synchronize()
    assert np.array_equal(lg.view(np.uint32), host(ref).view(np.uint32))
    assert np.array_equal(ids, host(rid))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,packed", [("f32", False), ("bf16", True)])
def test_zero_initialised_blocks_leave_h_unchanged(dtype, packed):
    m = lib()
    B, hd, V, K, topk, nb = 2, 256, 1500, 3, 5, 3
    h, w1, b1, w2, g, be = _inputs(dtype, B, hd, V, K, nb, True, seed=9)
    w1 = np.zeros_like(w1)
    b1 = np.zeros_like(b1)
    say("heads_ex zero init", dtype, packed)
    lg3, _ = _run(m, h, w1, b1, w2, g, be, dtype, packed, V, K, nb, topk)
    lg1, _ = _run(m, h, w1[:, :1], b1[:, :1], w2, None, None, dtype, packed, V, K, 1, topk)
    assert np.array_equal(lg3.view(np.uint32), lg1.view(np.uint32))
