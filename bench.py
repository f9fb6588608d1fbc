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
ceiling measured in the same run, accepted tokens/s, the fp64 CPU oracle timed on the host's own
cores (at the OpenMP thread count in force and at one thread), and a shorter measurement of the
same kind for every other workload ("all_configs").
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
# timed steps of the shorter per-workload measurement (all_configs), by workload index
LIGHT_STEPS = {0: 100, 1: 100, 2: 40, 3: 40, 4: 15}


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=1, help="workload index (0..4)")
    p.add_argument("--temperature", type=float, default=None)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time spent timing the oracle at the full thread count on the "
                        "headline workload (0 disables every oracle timing)")
    p.add_argument("--no-all-configs", dest="all_configs", action="store_false",
                   help="skip the shorter measurement of the other workloads")
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
        # top-k (the logits re-read, the ids written) and, in the same launch, the tree gather
        # (tokens and position ids written)
        "topk": B * K * V * 4 + B * K * cfg.topk * 4 + B * T * 8,
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


# ---------------------------------------------------------------------------------------------
# The fp64 oracle, timed on the host's cores
# ---------------------------------------------------------------------------------------------
def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    omp = int(os.environ.get("OMP_NUM_THREADS", affinity or 1))
    return {"cpu_model": model, "nproc": affinity, "os_cpu_count": os.cpu_count(),
            "omp_threads": omp}


class OracleInputs:
    """Host copies of one workload's inputs, the same seeded tensors the GPU step reads."""

    def __init__(self, cfg, choices, hin, logits):
        import oracle
        from synth import gen_attention_inputs, gen_root_tokens
        self.cfg, self.choices, self.hin, self.logits = cfg, choices, hin, logits
        self.st = oracle.build_static(choices, cfg.topk, cfg.K)
        self.a = gen_attention_inputs(cfg, self.st["T"])
        self.root = gen_root_tokens(cfg)


def oracle_whole_steps(inp, temperature, threads, seconds, min_steps):
    """Whole oracle steps (heads + top-k, tree, attention over every (b, q head, node) unit,
    typical acceptance) until `seconds` have passed and at least `min_steps` ran."""
    import oracle
    from oracle import _clib
    cfg, hin, a = inp.cfg, inp.hin, inp.a
    used = _clib.set_threads(threads)
    n, t0 = 0, time.perf_counter()
    while True:
        _, l64 = oracle.heads(hin["h"], hin["w1"], hin["b1"], hin["w2"], cfg.dtype)
        ids, _ = oracle.topk(l64, cfg.topk)
        st = oracle.build_static(inp.choices, cfg.topk, cfg.K)
        tokens, _ = oracle.gather(st, ids, inp.root, a["prefix_len"])
        oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, a["prefix_len"],
                              st["mask"], cfg.Hkv)
        oracle.typical_accept(inp.logits, cfg.dtype, tokens, st, temperature, cfg.eps, cfg.delta)
        n += 1
        if time.perf_counter() - t0 >= seconds and n >= min_steps:
            break
    dt = time.perf_counter() - t0
    return {"steps_per_s": n / dt, "threads": used,
            "sample": f"{n} whole steps in {dt:.1f} s"}


def oracle_staged(inp, temperature, threads, w2_frac=16, max_units=96):
    """One oracle step timed stage by stage on bounded samples, each scaled linearly to the whole
    stage: W1 and its epilogue whole; W2 on 1/w2_frac of the first head's vocab rows, scaled by
    the vocab and the head count (the projection costs the same per row); top-k (over logits of
    the same shape) and the tree whole; attention on max_units of the
    (b, q head, node) units (every unit reads the whole prefix); typical acceptance whole."""
    import oracle
    from oracle import _clib
    from synth.gen import rng_for
    cfg, hin, a, st = inp.cfg, inp.hin, inp.a, inp.st
    used = _clib.set_threads(threads)
    T = st["T"]
    t = {}
    t0 = time.perf_counter()
    r, _ = oracle.heads(hin["h"], hin["w1"], hin["b1"], np.ascontiguousarray(hin["w2"][:, :1]),
                        cfg.dtype)
    t["w1"] = time.perf_counter() - t0
    vs = max(1, cfg.V // w2_frac)
    w2s = np.ascontiguousarray(hin["w2"][0, :vs])
    t0 = time.perf_counter()
    oracle.project(w2s, cfg.dtype, np.ascontiguousarray(r[:, 0]))
    t["w2"] = (time.perf_counter() - t0) * (cfg.V / vs) * cfg.K
    l64 = np.random.default_rng(0).standard_normal((cfg.B, cfg.K, cfg.V))
    t0 = time.perf_counter()
    ids, _ = oracle.topk(l64, cfg.topk)
    st2 = oracle.build_static(inp.choices, cfg.topk, cfg.K)
    tokens, _ = oracle.gather(st2, ids, inp.root, a["prefix_len"])
    t["topk_tree"] = time.perf_counter() - t0
    units = cfg.B * cfg.Hq * T
    rng = rng_for(5, 9)
    n_sel = min(units, max_units)
    flat = np.sort(rng.choice(units, size=n_sel, replace=False))
    sel = np.stack([flat // (cfg.Hq * T), (flat // T) % cfg.Hq, flat % T], 1).astype(np.int32)
    t0 = time.perf_counter()
    oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, a["prefix_len"],
                          st["mask"], cfg.Hkv, sel=sel)
    t["attention"] = (time.perf_counter() - t0) * units / n_sel
    t0 = time.perf_counter()
    oracle.typical_accept(inp.logits, cfg.dtype, tokens, st2, temperature, cfg.eps, cfg.delta)
    t["accept"] = time.perf_counter() - t0
    total = sum(t.values())
    return {"steps_per_s": 1.0 / total, "threads": used,
            "stage_s": {k: round(v, 4) for k, v in t.items()},
            "sample": f"one step by stages: W2 on 1/{w2_frac} of the vocab rows and attention on "
                      f"{n_sel} of {units} units, each scaled to the whole stage"}


# ---------------------------------------------------------------------------------------------
# One workload resident on the GPU
# ---------------------------------------------------------------------------------------------
class Workload:
    def __init__(self, m, torch, cfg, keep_host=False):
        from synth import (gen_attention_inputs, gen_head_inputs, gen_root_tokens,
                           gen_verif_logits, load_tree_choices)
        self.m, self.torch, self.cfg = m, torch, cfg
        self.choices = load_tree_choices(cfg.tree)
        hin = gen_head_inputs(cfg)
        self.h, w1, self.b1, w2 = (self.dev(hin[k]) for k in ("h", "w1", "b1", "w2"))
        self.hin = hin if keep_host else None
        del hin
        if cfg.dtype == "bf16":
            # one-time repack of the static weights into the matrix-core operand order
            self.w1, self.w2 = m.pack_weights(w1), m.pack_weights(w2)
            del w1, w2
        else:
            self.w1, self.w2 = w1, w2
        torch.cuda.synchronize()
        self.step = m.VerifyStep(B=cfg.B, hidden=cfg.Hd, vocab=cfg.V, K=cfg.K, topk=cfg.topk,
                                 choices=self.choices, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D,
                                 max_prefix_len=cfg.L)
        self.T = self.step.tree.T
        self.n_int = self.step.tree.dims["n_internal"]
        a = gen_attention_inputs(cfg, self.T)
        self.q, self.kc, self.vc = self.dev(a["q"]), self.dev(a["k_cache"]), self.dev(a["v_cache"])
        self.pl = self.dev(a["prefix_len"])
        self.root = self.dev(gen_root_tokens(cfg))
        self.out = torch.empty_like(self.q)
        del a
        # the verification logits depend on this step's tree tokens: take them from one untimed
        # step
        self.step.heads(self.h, self.w1, self.b1, self.w2)
        self.step.build(self.root, self.pl)
        torch.cuda.synchronize()
        parent = self.step.tree.parent.cpu().numpy()
        logits = gen_verif_logits(cfg, parent, self.step.tokens.cpu().numpy())
        self.logits_host = logits if keep_host else None
        self.logits = self.dev(logits)
        del logits
        self.stream = torch.cuda.current_stream()

    def dev(self, a):
        t = self.torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
        t = t.cuda()
        return t.view(self.torch.bfloat16) if a.dtype == np.uint16 else t

    def run_kwargs(self, temp):
        cfg = self.cfg
        return dict(h=self.h, w1=self.w1, b1=self.b1, w2=self.w2, root_tokens=self.root,
                    prefix_len=self.pl, q=self.q, k_cache=self.kc, v_cache=self.vc,
                    attn_out=self.out, verif_logits=self.logits, temperature=temp,
                    eps=cfg.eps, delta=cfg.delta)

    def run(self, temp):
        self.step.run(**self.run_kwargs(temp))

    def timed_graph(self, temp, steps, warmup):
        """The same steps replayed from a HIP graph of one step (VerifyStep.capture): one host
        call per step.  Returns {steps_per_s, ms_per_step}, or the error if capture failed."""
        torch = self.torch
        try:
            graph = self.step.capture(**self.run_kwargs(temp))
        except Exception as e:          # reported, not fatal: the eager figures stand alone
            return {"error": f"{type(e).__name__}: {e}"}
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del graph
        return {"steps_per_s": round(steps / dt, 2), "ms_per_step": round(dt / steps * 1e3, 5)}

    def make_events(self, n):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for e0, e1 in ev:                  # create the underlying HIP events
            e0.record(self.stream)
            e1.record(self.stream)
        return ev

    def timed(self, temp, steps, warmup):
        """Whole steps back to back; every launch of the vocab projection bracketed by events.
        Returns (seconds, mean W2 launch ms)."""
        m, torch = self.m, self.torch
        w2_events = self.make_events(steps)
        for _ in range(warmup):
            self.run(temp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            m.set_kernel_events("heads_w2", *w2_events[i])
            self.run(temp)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        m.set_kernel_events("heads_w2", None, None)
        return t1 - t0, float(np.mean([e0.elapsed_time(e1) for e0, e1 in w2_events]))

    def kernel_pass(self, temp, nb, names, extra=None):
        """Mean ms of every launch of each named kernel over nb steps (every kernel bracketed by
        events, which slows the step: not a headline figure)."""
        m, torch = self.m, self.torch
        events = {k: self.make_events(nb) for k in names}
        for i in range(nb):
            for k in names:
                m.set_kernel_events(k, *events[k][i])
            self.run(temp)
            if extra is not None:
                extra()
        torch.cuda.synchronize()
        for k in names:
            m.set_kernel_events(k, None, None)
        return events

    def kernel_names(self):
        # the step's heads and tree run as one call, whose top-k merge also writes the tree
        # tokens: "topk" times top-k and the gather together
        names = ["heads_w1", "heads_w2", "topk", "attention", "accept"]
        if self.step.ws_attn.numel() > 256:
            names.insert(4, "attn_combine")
        return names


def summarize_kernels(cfg, w, events, kb):
    kernels = {}
    for k, evs in events.items():
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        ent = {"ms": round(ms, 5)}
        if k in kb:
            ent["alg_bytes"] = kb[k]
            ent["GB/s"] = round(kb[k] / (ms * 1e-3) / 1e9, 1)
            ent["hbm_frac"] = round(kb[k] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        kernels[k] = ent
    flops, anc = attention_flops(cfg, w.T, w.step.tree.mask.cpu().numpy())
    att = kernels["attention"]
    att["alg_flops"] = flops
    att["TFLOP/s"] = round(flops / (att["ms"] * 1e-3) / 1e12, 2)
    if cfg.dtype == "bf16":
        att["mfma_frac"] = round(att["TFLOP/s"] / MFMA_BF16_PEAK_TFLOPS, 4)
    else:
        att["valu_frac"] = round(att["TFLOP/s"] / FP32_VALU_PEAK_TFLOPS, 4)
    return kernels, anc


def measure_light(m, torch, ci, oracle_on, cpu_threads):
    """The shorter measurement of one workload: timed steps, the W2 launch rate, a per-kernel
    pass, greedy steps where the workload has temperature 0, and the oracle at the full thread
    count and at one thread."""
    from synth import get_config
    cfg = get_config(ci)
    temperature = cfg.temps[-1]
    w = Workload(m, torch, cfg, keep_host=oracle_on)
    steps = LIGHT_STEPS[ci]
    dt, w2_ms = w.timed(temperature, steps, warmup=5)
    alen = w.step.accept_length.cpu().numpy()
    kb = kernel_bytes(cfg, w.T, w.n_int)
    events = w.kernel_pass(temperature, 10, w.kernel_names())
    kernels, _ = summarize_kernels(cfg, w, events, kb)
    sps = steps / dt
    rec = {"workload": cfg.name, "batch": cfg.B, "tree_tokens": w.T, "prefix_len": cfg.L,
           "temperature": temperature, "steps": steps, "steps_per_s": round(sps, 2),
           "ms_per_step": round(dt / steps * 1e3, 5), "accept_length": alen.tolist(),
           "accepted_tokens_per_s": round(sps * int((alen + 1).sum()), 1),
           "w2": {"avg_launch_ms": round(w2_ms, 5),
                  "GB/s": round(kb["heads_w2"] / (w2_ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(kb["heads_w2"] / (w2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "kernels": kernels, "graph": w.timed_graph(temperature, steps, 5)}
    if cfg.temps[0] == 0.0 and temperature != 0.0:
        dt0, _ = w.timed(0.0, max(5, steps // 2), warmup=2)
        a0 = w.step.accept_length.cpu().numpy()
        n0 = max(5, steps // 2)
        rec["greedy"] = {"steps_per_s": round(n0 / dt0, 2), "accept_length": a0.tolist(),
                         "accepted_tokens_per_s": round(n0 / dt0 * int((a0 + 1).sum()), 1)}
    if oracle_on:
        inp = OracleInputs(cfg, w.choices, w.hin, w.logits_host)
        del w
        torch.cuda.empty_cache()
        rec["oracle"] = oracle_rates(inp, temperature, cpu_threads, ci)
    return rec


def oracle_rates(inp, temperature, cpu_threads, ci, seconds=3.0):
    """The oracle at the full thread count and at one thread: whole steps on the two small
    workloads, stage samples on the three large ones (their whole steps take minutes at one
    thread)."""
    out = {}
    for label, th in (("threads_n", cpu_threads), ("threads_1", 1)):
        if ci <= 1:
            r = oracle_whole_steps(inp, temperature, th, seconds, 1)
        else:
            r = oracle_staged(inp, temperature, th)
        r["steps_per_s"] = round(r["steps_per_s"], 4)
        out[label] = r
    return out


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
    from synth import get_config

    cfg = get_config(args.config)
    temperature = args.temperature if args.temperature is not None else cfg.temps[-1]
    oracle_on = args.cpu_seconds > 0
    info = host_info()
    w = Workload(m, torch, cfg, keep_host=oracle_on)
    step, T, n_int, stream = w.step, w.T, w.n_int, w.stream
    run = w.run

    # ---- timed region: whole steps; the dominant kernel is bracketed by HIP events ----
    dt, w2_ms = w.timed(temperature, args.steps, args.warmup)
    steps_per_s = args.steps / dt
    alen = step.accept_length.cpu().numpy()
    emitted = int((alen + 1).sum())

    # ---- per-kernel breakdown: a separate pass with every kernel bracketed by events (the
    #      extra event records slow the step, so this pass is not the headline) ----
    #      The commit of the accepted candidate (the decode-loop glue after the step) is timed
    #      here too, on copies of the caches so that the step's inputs stay fixed. ----
    names = w.kernel_names() + ["commit"]
    kc_commit, vc_commit = w.kc.clone(), w.vc.clone()
    nb = max(10, min(args.steps, 50))
    events = w.kernel_pass(temperature, nb, names,
                           extra=lambda: step.commit(kc_commit, vc_commit, w.pl))
    del kc_commit, vc_commit
    # the rotary-embedding variant of tree attention, on a copy of the cache (it rotates the tree
    # key rows in place): its key-rotation kernel ("rope") and its attention kernel, which
    # rotates the queries as it loads them ("attention_rope")
    kc_rope = w.kc.clone()
    out_rope = torch.empty_like(w.out)
    ws_rope = m.workspace(m.tree_attention_rope_workspace(cfg.B, cfg.Hq, cfg.Hkv, T, cfg.D, cfg.L))
    events["rope"] = w.make_events(nb)
    events["attention_rope"] = w.make_events(nb)
    for i in range(nb):
        m.set_kernel_events("rope", *events["rope"][i])
        m.set_kernel_events("attention", *events["attention_rope"][i])
        m.tree_attention_rope(w.q, kc_rope, w.vc, w.pl, cfg.L, step.tree.mask, step.position_ids,
                              out_rope, ws_rope)
    torch.cuda.synchronize()
    m.set_kernel_events("rope", None, None)
    m.set_kernel_events("attention", None, None)
    del kc_rope, out_rope, ws_rope
    # the nucleus mode of evaluate_posterior (top_p 0.9) on the step's logits and tree tokens,
    # its three acceptance launches together ("accept_nucleus"; at temperature 0 both modes are
    # the greedy one, so it runs at 0.7 there)
    ws_nuc = m.workspace(m.evaluate_posterior_workspace(cfg.B, cfg.V, step.tree, "nucleus"))
    nuc_out = [torch.empty((cfg.B,), dtype=torch.int32, device="cuda") for _ in range(3)]
    nuc_temp = temperature if temperature > 0 else 0.7
    events["accept_nucleus"] = w.make_events(nb)
    for i in range(nb):
        m.set_kernel_events("accept", *events["accept_nucleus"][i])
        m.evaluate_posterior(w.logits, step.tokens, step.tree, nuc_temp, cfg.eps, cfg.delta,
                             nuc_out[0], nuc_out[1], ws_nuc, top_p=0.9, sampling="nucleus",
                             next_token=nuc_out[2])
    torch.cuda.synchronize()
    m.set_kernel_events("accept", None, None)
    del ws_nuc, nuc_out
    kb = kernel_bytes(cfg, T, n_int)
    # rope: every tree key row read and written once, and each node's cos/sin written (fp32);
    # attention_rope: the attention's bytes plus that table, read once
    kb["rope"] = 2 * cfg.B * cfg.Hkv * T * cfg.D * cfg.esize + cfg.B * T * cfg.D * 4
    kb["attention_rope"] = kb["attention"] + cfg.B * T * cfg.D * 4
    kb["accept_nucleus"] = kb["accept"]
    # commit: each accepted node's K and V rows read and written once, plus the emitted tokens
    moved = int(step.accept_length.cpu().numpy().sum())
    kb["commit"] = 4 * moved * cfg.Hkv * cfg.D * cfg.esize + cfg.B * (step.tree.dims["dmax"] + 1) * 4
    kernels, anc = summarize_kernels(cfg, w, events, kb)

    # ---- per-step distribution, back to back (warm) and with the 256 MB MALL flushed by a
    #      1 GiB write before every step (cold; the flush is outside the step's events) ----
    def per_step(n, flush=None):
        ev = w.make_events(n)
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
    graph_rate = w.timed_graph(temperature, args.steps, 5)
    flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    cold = per_step(nd, flush)
    del flush

    # ---- measured streaming-read ceiling: the library's plain read kernel over 4 GiB ----
    buf = torch.zeros(CEILING_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    cev = w.make_events(10)
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
    xev = w.make_events(20)
    for i in range(22):
        if i >= 2:
            xev[i - 2][0].record(stream)
        m.medusa_heads_ex(w.h, w1x, b1x, w.w2, cfg.V, cfg.K, nbx, cfg.topk, idsx, wsx, ln_gamma=gx,
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
        dt0, _ = w.timed(0.0, n0, warmup=3)
        a0 = step.accept_length.cpu().numpy()
        t0g = {"steps_per_s": round(n0 / dt0, 2),
               "accept_length": a0.tolist(),
               "accepted_tokens_per_s": round(n0 / dt0 * int((a0 + 1).sum()), 1)}

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

    headline_summary = {
        "workload": cfg.name, "batch": cfg.B, "tree_tokens": T, "prefix_len": cfg.L,
        "temperature": temperature, "steps": args.steps, "steps_per_s": round(steps_per_s, 2),
        "ms_per_step": round(dt / args.steps * 1e3, 5), "accept_length": alen.tolist(),
        "accepted_tokens_per_s": round(steps_per_s * emitted, 1),
        "w2": {"avg_launch_ms": round(w2_ms, 5), "GB/s": roofline["achieved"],
               "hbm_frac": roofline["frac"]},
        "kernels": {k: kernels[k] for k in w.kernel_names()}, "graph": graph_rate, "greedy": t0g}

    # ---- the oracle on the host's cores: whole steps at the OpenMP thread count in force (the
    #      headline baseline), then at one thread ----
    cpu = None
    if oracle_on:
        inp = OracleInputs(cfg, w.choices, w.hin, w.logits_host)
        del w, step, run
        torch.cuda.empty_cache()
        ci = args.config
        big = ci >= 2
        if big:
            rn = oracle_staged(inp, temperature, info["omp_threads"])
            r1 = oracle_staged(inp, temperature, 1)
        else:
            rn = oracle_whole_steps(inp, temperature, info["omp_threads"], args.cpu_seconds, 2)
            r1 = oracle_whole_steps(inp, temperature, 1, min(args.cpu_seconds, 5.0), 1)
        cpu = {"value": rn["steps_per_s"], "unit": "steps/s", "cores": rn["threads"],
               "kind": "oracle",
               "sample": f"{rn['sample']} of the same workload (heads + top-k, tree, attention "
                         f"over all {cfg.B * cfg.Hq * T} (b, q head, node) units, typical "
                         f"acceptance), fp64, inputs in host memory, {rn['threads']} OpenMP "
                         f"threads",
               "one_thread": {"value": r1["steps_per_s"], "unit": "steps/s", "cores": 1,
                              "sample": r1["sample"]},
               **{k: info[k] for k in ("cpu_model", "nproc", "os_cpu_count")}}
        headline_summary["oracle"] = {"threads_n": rn, "threads_1": r1}
        del inp
    else:
        del w, step, run
        torch.cuda.empty_cache()

    # ---- the shorter measurement of every other workload ----
    all_configs = None
    if args.all_configs:
        all_configs = {}
        for ci in range(5):
            if ci == args.config:
                all_configs[f"c{ci}"] = headline_summary
                continue
            all_configs[f"c{ci}"] = measure_light(m, torch, ci, oracle_on, info["omp_threads"])
            torch.cuda.empty_cache()

    # the step's own kernels (not the rotary and commit kernels timed beside it)
    total_bytes = sum(kernel_bytes(cfg, T, n_int).values())
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
        "graph_replay": graph_rate,
        "step_time_mall_flushed": cold,
        "tree": {"ancestors_or_self": anc, "internal_rows": n_int,
                 "sparse_tree_host_us": round(sparse_us, 1),
                 "sparse_tree_expected_accept_length": round(exp_len, 4)},
        "greedy": t0g,
        "all_configs": all_configs,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
