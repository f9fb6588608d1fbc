#!/usr/bin/env python3
"""Throughput of one Medusa verification step on one MI355X.

A step is the whole hot path on one batch of synthetic inputs already resident in HBM:
medusa_heads (K heads + per-head top-k) -> build_tree (tokens, position ids) -> tree_attention
-> typical_accept (best path, accept length, next token).  Default workload: the Vicuna-7B shape
(hidden 4096, vocab 32000, 4 heads, top-10, a 64-node sparse tree, 32 heads x 128 attention over
a 1024-token prefix, bf16, temperature 0.7).

Prints one JSON line: steps/s, the roofline of the dominant kernel (the heads' vocab
projection, timed per launch with HIP events recorded around it on its own stream), per-kernel
timings with their HBM (and, for attention, matrix-core) fractions, the per-step median and
p10/p90 back to back and with the last-level cache flushed before every step, a streaming-read
ceiling measured in the same run, accepted tokens/s, and the fp64 CPU oracle timed on a bounded
sample of the same step.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix cores
FP32_VALU_PEAK_TFLOPS = 157.3    # fp32 vector ALUs
MALL_FLUSH_BYTES = 1 << 30       # written before each cold step: 4x the 256 MB last-level cache
CEILING_BYTES = 4 << 30          # buffer read by the streaming-read ceiling kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "heads_w2_vicuna7b_traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=1, help="workload index (0..4)")
    p.add_argument("--temperature", type=float, default=None)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time spent timing the oracle (0 disables it)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy 3x (untimed), the reference kernel "
                        "for scaling hardware byte counters")
    return p.parse_args()


def kernel_bytes(cfg, T, n_int):
    """Algorithmic HBM bytes per launch of each kernel (what the method must read or write)."""
    s = cfg.esize
    B, K, Hd, V = cfg.B, cfg.K, cfg.Hd, cfg.V
    return {
        "heads_w1": K * Hd * Hd * s + K * Hd * s + B * Hd * s + B * K * Hd * 4,
        "heads_w2": K * V * Hd * s + B * K * Hd * 4 + B * K * V * 4,
        "topk": B * K * V * 4 + B * K * cfg.topk * 4,
        "tree_gather": B * T * 8 + B * K * cfg.topk * 4,
        "attention": 2 * B * cfg.Hkv * (cfg.L + T) * cfg.D * s + 2 * B * cfg.Hq * T * cfg.D * s,
        "accept": B * n_int * V * s,
    }


def attention_flops(cfg, T, mask):
    """Algorithmic flops of one tree_attention call: 2 flops per multiply-add of QK^T and of PV
    over the visible columns only (every prefix column, plus each node's ancestors-or-self)."""
    anc = int(np.unpackbits(np.ascontiguousarray(mask).view(np.uint8)).sum())
    return 4 * cfg.D * cfg.B * cfg.Hq * (T * cfg.L + anc), anc


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic():
    """HBM bytes per launch of the vocab-projection kernel from committed rocprofv3 counter runs,
    or None if they are missing or the kernel source changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    src = os.path.join(ROOT, "medusa_head_speculative_amd", "csrc", "heads.hip")
    if t.get("source_sha256") != source_digest(src):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(cfg, choices, temperature, seconds):
    """The fp64 oracle, as it stands, on whole steps of the same workload (inputs in host RAM)."""
    import oracle
    from synth import (gen_attention_inputs, gen_head_inputs, gen_root_tokens, gen_verif_logits)
    hin = gen_head_inputs(cfg)
    st = oracle.build_static(choices, cfg.topk, cfg.K)
    a = gen_attention_inputs(cfg, st["T"])
    root = gen_root_tokens(cfg)

    def one_step():
        _, l64 = oracle.heads(hin["h"], hin["w1"], hin["b1"], hin["w2"], cfg.dtype)
        ids, _ = oracle.topk(l64, cfg.topk)
        stt = oracle.build_static(choices, cfg.topk, cfg.K)
        tokens, _ = oracle.gather(stt, ids, root, a["prefix_len"])
        oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, a["prefix_len"],
                              stt["mask"], cfg.Hkv)
        return stt, tokens

    stt, tokens = one_step()
    logits = gen_verif_logits(cfg, stt["parent"], np.array(tokens))
    n, t0 = 0, time.perf_counter()
    while True:
        stt, tokens = one_step()
        oracle.typical_accept(logits, cfg.dtype, tokens, stt, temperature, cfg.eps, cfg.delta)
        n += 1
        if time.perf_counter() - t0 >= seconds and n >= 2:
            break
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": n / dt, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} whole verification steps of the same workload (heads + top-k, tree, "
                      f"attention over all {cfg.B * cfg.Hq * st['T']} (b, q head, node) rows, "
                      f"typical acceptance), fp64, inputs in host memory, {dt:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit(f"bench.py runs on exactly one GPU: this build has no multi-GPU path "
                 f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).")
    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    import medusa_head_speculative_amd as m
    if not os.path.exists(m._lib.LIBPATH):
        from medusa_head_speculative_amd import build
        build.build()
    m.load()
    from synth import (gen_attention_inputs, gen_head_inputs, gen_root_tokens, gen_verif_logits,
                       get_config, load_tree_choices)

    cfg = get_config(args.config)
    temperature = args.temperature if args.temperature is not None else cfg.temps[-1]
    choices = load_tree_choices(cfg.tree)

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
        t = t.cuda()
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    hin = gen_head_inputs(cfg)
    h, w1, b1, w2 = (dev(hin[k]) for k in ("h", "w1", "b1", "w2"))
    del hin
    if cfg.dtype == "bf16":
        # one-time repack of the static weights into the matrix-core operand order
        w1, w2 = m.pack_weights(w1), m.pack_weights(w2)
        torch.cuda.synchronize()
    step = m.VerifyStep(B=cfg.B, hidden=cfg.Hd, vocab=cfg.V, K=cfg.K, topk=cfg.topk,
                        choices=choices, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, max_prefix_len=cfg.L)
    T = step.tree.T
    n_int = step.tree.dims["n_internal"]
    a = gen_attention_inputs(cfg, T)
    q, kc, vc = dev(a["q"]), dev(a["k_cache"]), dev(a["v_cache"])
    pl = dev(a["prefix_len"])
    root = dev(gen_root_tokens(cfg))
    out = torch.empty_like(q)
    # the verification logits depend on this step's tree tokens: take them from one untimed step
    step.heads(h, w1, b1, w2)
    step.build(root, pl)
    torch.cuda.synchronize()
    parent = step.tree.parent.cpu().numpy()
    logits = dev(gen_verif_logits(cfg, parent, step.tokens.cpu().numpy()))

    def run(temp):
        step.run(h=h, w1=w1, b1=b1, w2=w2, root_tokens=root, prefix_len=pl, q=q, k_cache=kc,
                 v_cache=vc, attn_out=out, verif_logits=logits, temperature=temp,
                 eps=cfg.eps, delta=cfg.delta)

    stream = torch.cuda.current_stream()

    def make_events(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for e0, e1 in ev:                  # create the underlying HIP events
            e0.record(stream)
            e1.record(stream)
        return ev

    # ---- timed region: whole steps; the dominant kernel is bracketed by HIP events ----
    w2_events = make_events(args.steps)
    for _ in range(args.warmup):
        run(temperature)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        m.set_kernel_events("heads_w2", *w2_events[i])
        run(temperature)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.set_kernel_events("heads_w2", None, None)
    dt = t1 - t0
    steps_per_s = args.steps / dt
    alen = step.accept_length.cpu().numpy()
    emitted = int((alen + 1).sum())
    w2_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in w2_events]))

    # ---- per-kernel breakdown: a separate pass with every kernel bracketed by events (the
    #      extra event records slow the step, so this pass is not the headline) ----
    #      The commit of the accepted candidate (the decode-loop glue after the step) is timed
    #      here too, on copies of the caches so that the step's inputs stay fixed. ----
    splits = step.ws_attn.numel() > 256
    names = ["heads_w1", "heads_w2", "topk", "tree_gather", "attention", "accept", "commit"]
    if splits:
        names.insert(5, "attn_combine")
    kc_commit, vc_commit = kc.clone(), vc.clone()
    nb = max(10, min(args.steps, 50))
    events = {k: make_events(nb) for k in names}
    for i in range(nb):
        for k in names:
            m.set_kernel_events(k, *events[k][i])
        run(temperature)
        step.commit(kc_commit, vc_commit, pl)
    torch.cuda.synchronize()
    del kc_commit, vc_commit
    for k in names:
        m.set_kernel_events(k, None, None)
    # the rotary-embedding variant of tree attention, on a copy of the cache (it rotates the tree
    # key rows in place): its key-rotation kernel ("rope") and its attention kernel, which
    # rotates the queries as it loads them ("attention_rope")
    kc_rope = kc.clone()
    out_rope = torch.empty_like(out)
    ws_rope = m.workspace(m.tree_attention_rope_workspace(cfg.B, cfg.Hq, cfg.Hkv, T, cfg.D, cfg.L))
    events["rope"] = make_events(nb)
    events["attention_rope"] = make_events(nb)
    for i in range(nb):
        m.set_kernel_events("rope", *events["rope"][i])
        m.set_kernel_events("attention", *events["attention_rope"][i])
        m.tree_attention_rope(q, kc_rope, vc, pl, cfg.L, step.tree.mask, step.position_ids,
                              out_rope, ws_rope)
    torch.cuda.synchronize()
    m.set_kernel_events("rope", None, None)
    m.set_kernel_events("attention", None, None)
    del kc_rope, out_rope, ws_rope
    kb = kernel_bytes(cfg, T, n_int)
    # rope: every tree key row read and written once, and each node's cos/sin written (fp32);
    # attention_rope: the attention's bytes plus that table, read once
    kb["rope"] = 2 * cfg.B * cfg.Hkv * T * cfg.D * cfg.esize + cfg.B * T * cfg.D * 4
    kb["attention_rope"] = kb["attention"] + cfg.B * T * cfg.D * 4
    # commit: each accepted node's K and V rows read and written once, plus the emitted tokens
    moved = int(step.accept_length.cpu().numpy().sum())
    kb["commit"] = 4 * moved * cfg.Hkv * cfg.D * cfg.esize + cfg.B * (step.tree.dims["dmax"] + 1) * 4
    kernels = {}
    for k, evs in events.items():
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        ent = {"ms": round(ms, 5)}
        if k in kb:
            ent["alg_bytes"] = kb[k]
            ent["GB/s"] = round(kb[k] / (ms * 1e-3) / 1e9, 1)
            ent["hbm_frac"] = round(kb[k] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        kernels[k] = ent

    # ---- per-step distribution, back to back (warm) and with the 256 MB MALL flushed by a
    #      1 GiB write before every step (cold; the flush is outside the step's events) ----
    def per_step(n, flush=None):
        ev = make_events(n)
        for i in range(n):
            if flush is not None:
                flush.fill_(i & 0x7F)
            ev[i][0].record(stream)
            run(temperature)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        return {"median_ms": round(float(np.median(t)), 5),
                "p10_ms": round(float(np.percentile(t, 10)), 5),
                "p90_ms": round(float(np.percentile(t, 90)), 5), "steps": n}

    nd = max(10, min(args.steps, 100))
    warm = per_step(nd)
    flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    cold = per_step(nd, flush)
    del flush

    # ---- measured streaming-read ceiling: the library's plain read kernel over 4 GiB ----
    buf = torch.zeros(CEILING_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    cev = make_events(10)
    for _ in range(2):
        m.stream_read(buf, sink)
    for e0, e1 in cev:
        e0.record(stream)
        m.stream_read(buf, sink)
        e1.record(stream)
    torch.cuda.synchronize()
    ceiling_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in cev]))
    ceiling_gbs = CEILING_BYTES / (ceiling_ms * 1e-3) / 1e9
    # the same plain read over exactly the vocab projection's weight bytes: a ceiling for one
    # launch of that size, start-up and drain included
    w2_weight_bytes = (cfg.K * cfg.V * cfg.Hd * cfg.esize) // 16 * 16
    same = buf[:w2_weight_bytes] if w2_weight_bytes <= CEILING_BYTES else None
    same_ms = None
    if same is not None:
        for e0, e1 in cev:
            e0.record(stream)
            m.stream_read(same, sink)
            e1.record(stream)
        torch.cuda.synchronize()
        same_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in cev]))
    del buf, sink, same
    for ent in kernels.values():
        if "GB/s" in ent:
            ent["ceiling_frac"] = round(ent["GB/s"] / ceiling_gbs, 4)
    flops, anc = attention_flops(cfg, T, step.tree.mask.cpu().numpy())
    att = kernels["attention"]
    att["alg_flops"] = flops
    att["TFLOP/s"] = round(flops / (att["ms"] * 1e-3) / 1e12, 2)
    if cfg.dtype == "bf16":
        att["mfma_frac"] = round(att["TFLOP/s"] / MFMA_BF16_PEAK_TFLOPS, 4)
    else:
        att["valu_frac"] = round(att["TFLOP/s"] / FP32_VALU_PEAK_TFLOPS, 4)

    # head variant: two residual blocks opened by LayerNorm at this workload's shape (random
    # weights drawn on the device), timed as whole medusa_heads_ex calls
    nbx = 2
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    std = cfg.Hd ** -0.5
    def rnd(*shape, scale=std, shift=0.0):
        return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * scale + shift).to(tdt)
    w1x = rnd(cfg.K * nbx, cfg.Hd, cfg.Hd)
    b1x, gx, bx = rnd(cfg.K, nbx, cfg.Hd), rnd(cfg.K, nbx, cfg.Hd, scale=0.1, shift=1.0), rnd(cfg.K, nbx, cfg.Hd, scale=0.1)
    packed = cfg.dtype == "bf16"
    if packed:
        w1x = m.pack_weights(w1x)
    else:
        w1x = w1x.view(cfg.K, nbx, cfg.Hd, cfg.Hd)
    wsx = m.workspace(m.medusa_heads_ex_workspace(cfg.B, cfg.Hd, cfg.V, cfg.K, nbx, True, cfg.topk))
    idsx = torch.zeros((cfg.B, cfg.K, cfg.topk), dtype=torch.int32, device="cuda")
    hx = h
    xev = make_events(20)
    for i in range(22):
        if i >= 2:
            xev[i - 2][0].record(stream)
        m.medusa_heads_ex(hx, w1x, b1x, w2, cfg.V, cfg.K, nbx, cfg.topk, idsx, wsx, ln_gamma=gx,
                          ln_beta=bx, packed=packed)
        if i >= 2:
            xev[i - 2][1].record(stream)
    torch.cuda.synchronize()
    x_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in xev]))
    x_bytes = cfg.K * (nbx * cfg.Hd * cfg.Hd + cfg.V * cfg.Hd) * cfg.esize
    head_variant = {"n_blocks": nbx, "layernorm": True, "ms": round(x_ms, 5), "alg_bytes": x_bytes,
                    "GB/s": round(x_bytes / (x_ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(x_bytes / (x_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del w1x, b1x, gx, bx, wsx

    # host-side construction of this workload's sparse tree from per-head rank accuracies
    # (the synthetic 60 % / 80 % model), for the record: it runs once per model, not per step
    acc = np.array([[0.6 * (r + 1) ** -2.35 for r in range(cfg.topk)]] * cfg.K)
    n_nodes = T - 1
    t_sp = time.perf_counter()
    for _ in range(20):
        _, exp_len = m.sparse_tree(acc, min(n_nodes, 4095))
    sparse_us = (time.perf_counter() - t_sp) / 20 * 1e6

    # greedy (temperature 0) for context: shorter run
    t0g = None
    if cfg.temps[0] == 0.0 and temperature != 0.0:
        n0 = max(10, args.steps // 4)
        for _ in range(3):
            run(0.0)
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for _ in range(n0):
            run(0.0)
        torch.cuda.synchronize()
        s1 = time.perf_counter()
        a0 = step.accept_length.cpu().numpy()
        t0g = {"steps_per_s": round(n0 / (s1 - s0), 2),
               "accept_length": a0.tolist(),
               "accepted_tokens_per_s": round(n0 / (s1 - s0) * int((a0 + 1).sum()), 1)}

    w2_bytes = kb["heads_w2"]
    achieved = w2_bytes / (w2_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(),
                "kernel": "heads_gemv_packed (vocab projection W2 of all heads, one launch)"
                          if cfg.dtype == "bf16" else "heads_gemv_f32 (vocab projection W2)",
                "alg_bytes_per_launch": w2_bytes, "avg_launch_ms": round(w2_ms, 5),
                "measured_read_ceiling_GB/s": round(ceiling_gbs, 1),
                "frac_of_measured_ceiling": round(achieved / ceiling_gbs, 4),
                "plain_read_same_weight_bytes_ms": None if same_ms is None else round(same_ms, 5),
                "frac_of_plain_read_same_bytes": None if same_ms is None else round(same_ms / w2_ms, 4)}

    if args.copy_calibration:
        src = torch.ones(128 << 20, dtype=torch.bfloat16, device="cuda")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, choices, temperature, args.cpu_seconds)

    total_bytes = sum(kb.values())
    rec = {
        "metric": "Medusa verify steps/s + tree-attn/head HBM GB/s (7B shape, 64-node tree)",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian weights/KV/logits of the workload's shapes)",
        "config": {"workload": f"{cfg.name}: one verification step, B={cfg.B}, hidden {cfg.Hd}, "
                               f"vocab {cfg.V}, {cfg.K} heads, top-{cfg.topk}, tree of {T} tokens "
                               f"({cfg.tree}), attention {cfg.Hq}q/{cfg.Hkv}kv heads x {cfg.D} "
                               f"over a {cfg.L}-token prefix, temperature {temperature}",
                   "batch": cfg.B, "tree_tokens": T, "prefix_len": cfg.L,
                   "temperature": temperature, "eps": cfg.eps, "delta": cfg.delta},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "accept_length": alen.tolist(),
        "accepted_tokens_per_s": round(steps_per_s * emitted, 1),
        "step_alg_bytes": total_bytes,
        "step_GB/s": round(total_bytes * steps_per_s / 1e9, 1),
        "kernels": kernels,
        "heads_variant": head_variant,
        "step_time_warm": warm,
        "step_time_mall_flushed": cold,
        "tree": {"ancestors_or_self": anc, "internal_rows": n_int,
                 "sparse_tree_host_us": round(sparse_us, 1),
                 "sparse_tree_expected_accept_length": round(exp_len, 4)},
        "greedy": t0g,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
