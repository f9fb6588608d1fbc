"""Helpers for the GPU tests: host <-> device transfer, library loading, parity comparisons."""

import itertools
import os
import sys

import numpy as np

import oracle
from oracle.accept import scan_paths


def say(*a):
    """Name the case before a GPU step (and flush), so a fault report points at it."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def lib():
    import medusa_head_speculative_amd as m
    so = os.path.join(os.path.dirname(m.__file__), "libmedusa_hip.so")
    if not os.path.exists(so):
        from medusa_head_speculative_amd import build
        build.build()
    m.load()
    return m


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(a, dtype):
    return bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, np.float64)


def tol(dtype):
    """Max-abs tolerance for head logits and attention outputs against the fp64 oracle."""
    return 1e-4 if dtype == "f32" else 2e-2


def sample_units(B, Hq, T, n, seed):
    """(b, q head, node) units at which a full-size attention output is compared with the
    oracle: every head of the first and the last sequence at a few nodes (the last sequence's
    units are the ones a work plan runs last), plus n random units."""
    from synth.gen import rng_for
    rng = rng_for(seed, 9)
    sel = [(b, h, i) for b in {0, B - 1} for h in range(Hq) for i in {0, 1, T // 2, T - 1}]
    sel += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(n)]
    return np.array(sorted(set(sel)), np.int32)


def attention_all_f32(q, kc, vc, prefix_len, mask_words, Hkv):
    """Every output of tree attention from plain float32 PyTorch ops on the device: node n of
    sequence b attends to the b's prefix rows and the tree rows its mask word selects, with
    softmax(q k^T / sqrt(D)) v (Wiblog, tree-attention section).  A test reference for checking
    all outputs at sizes the fp64 oracle can only sample; tests pin it to the oracle on the
    sampled units first.  Returns float64 [B, Hq, T, D]."""
    import torch
    torch.backends.cuda.matmul.allow_tf32 = False
    B, Hq, T, D = q.shape
    G = Hq // Hkv
    words = np.ascontiguousarray(np.asarray(mask_words, np.uint64).reshape(T, -1))
    bits = np.unpackbits(words.view(np.uint8), axis=1, bitorder="little")[:, :T].astype(bool)
    vis_tree = torch.from_numpy(bits).cuda()
    qd, kd, vd = dev(q).float(), dev(kc).float(), dev(vc).float()
    out = torch.empty((B, Hq, T, D), dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        L = int(prefix_len[b])
        vis = torch.cat([torch.ones((T, L), dtype=torch.bool, device="cuda"), vis_tree], 1)
        for g in range(Hkv):
            k = kd[b, g, :L + T].contiguous()
            v = vd[b, g, :L + T].contiguous()
            qq = qd[b, g * G:(g + 1) * G].reshape(G * T, D).contiguous()
            s = (qq @ k.t().contiguous()) * scale
            s = s.view(G, T, L + T).masked_fill(~vis.unsqueeze(0), float("-inf"))
            p = torch.softmax(s, dim=-1).reshape(G * T, L + T)
            out[b, g * G:(g + 1) * G] = (p @ v).view(G, T, D)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def mask_array(static):
    return np.array(static["mask"], dtype=np.uint64)


def check_topk(gpu_ids, logits64, k, rel=1e-4):
    """Top-k ids must equal the oracle's bit for bit, except rows with a top-k tie, where the
    GPU ids must hold the same values up to the tie tolerance.  Returns (#rows, #tie rows)."""
    ids64, vals64 = oracle.topk(logits64, k)
    ties = oracle.topk_ties(logits64, k, rel)
    flat_g = gpu_ids.reshape(-1, k)
    flat_o = ids64.reshape(-1, k)
    flat_t = ties.reshape(-1)
    flat_l = logits64.reshape(-1, logits64.shape[-1])
    for r in range(flat_g.shape[0]):
        if not flat_t[r]:
            assert flat_g[r].tolist() == flat_o[r].tolist(), (r, flat_g[r], flat_o[r])
        else:
            gv = np.sort(flat_l[r][flat_g[r]])[::-1]
            ov = np.sort(vals64.reshape(-1, k)[r])[::-1]
            assert len(set(flat_g[r].tolist())) == k
            np.testing.assert_allclose(gv, ov, rtol=0, atol=2 * rel * max(1.0, abs(ov[0])))
    return flat_g.shape[0], int(flat_t.sum())


def accept_candidates(static, res, logits, dtype, band=1e-4, max_flips=10):
    """All (best, accept_length, next_token) results the method allows for each sequence given
    fp64-vs-fp32 uncertainty: decisions with |ln p - ln thr| <= band on nodes whose ancestors are
    all accepted may go either way.  Returns a list (per b) of sets, and the banded count."""
    B, T = res["accepted"].shape
    out, nband = [], 0
    for b in range(B):
        acc = res["accepted"][b].copy()
        live = []
        for c in range(1, T):
            m = res["margin"][b, c]
            if not np.isnan(m) and abs(m) <= band:
                j, ok = static["parent"][c], True
                while j > 0:
                    ok &= bool(acc[j])
                    j = static["parent"][j]
                if ok:
                    live.append(c)
        nband += len(live)
        live = live[:max_flips]
        cands = set()
        for bits in itertools.product([False, True], repeat=len(live)):
            a = acc.copy()
            for c, flip in zip(live, bits):
                if flip:
                    a[c] = not a[c]
            best, alen, last = scan_paths(static, a)
            row = as_f64(logits[b, last], dtype)
            cands.add((best, alen, int(np.flatnonzero(row == row.max())[0])))
        out.append(cands)
    return out, nband
