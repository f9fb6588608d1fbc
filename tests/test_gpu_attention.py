"""GPU parity of tree_attention against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
from gpu_util import (as_f64, attention_all_f32, dev, host, lib, mask_array, sample_units,
                      say, tol)
from synth import gen_attention_inputs, get_config
from synth.configs import custom
from synth.gen import rng_for
from synth.trees import cartesian_choices, load_tree_choices

pytestmark = pytest.mark.gpu


def run_attn(m, a, mask, Hkv, max_pl=None):
    import torch
    q = dev(a["q"])
    B, Hq, T, D = q.shape
    max_pl = int(a["prefix_len"].max()) if max_pl is None else max_pl
    out = torch.full_like(q, float("nan"))
    ws = m.workspace(m.tree_attention_workspace(B, Hq, Hkv, T, D, max_pl))
    m.tree_attention(q, dev(a["k_cache"]), dev(a["v_cache"]), dev(a["prefix_len"]), max_pl,
                     dev(mask.view(np.int64)), out, ws)
    torch.cuda.synchronize()
    return host(out)


def _sample_units(B, Hq, T, n, seed):
    return sample_units(B, Hq, T, n, seed)


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_attention_full_size(ci):
    cfg = get_config(ci)
    m = lib()
    st = oracle.build_static(load_tree_choices(f"c{ci}"), cfg.topk, cfg.K)
    T = st["T"]
    a = gen_attention_inputs(cfg, T)
    mask = mask_array(st)
    say("attention full size", cfg.name, dict(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, T=T, L=cfg.L))
    out = run_attn(m, a, mask, cfg.Hkv)
    full = ci <= 2
    sel = None if full else _sample_units(cfg.B, cfg.Hq, T, 400, ci)
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], cfg.dtype, a["prefix_len"],
                                st["mask"], cfg.Hkv, sel=sel)
    got = as_f64(out, cfg.dtype)
    assert not np.isnan(got).any()
    if sel is not None:
        # every output against a float32 device reference, itself pinned to the oracle on the
        # sampled units
        every = attention_all_f32(a["q"], a["k_cache"], a["v_cache"], a["prefix_len"], mask, cfg.Hkv)
        ref = ref[sel[:, 0], sel[:, 1], sel[:, 2]]
        pin = float(np.abs(every[sel[:, 0], sel[:, 1], sel[:, 2]] - ref).max())
        assert pin <= 1e-4, pin
        err_all = float(np.abs(got - every).max())
        print(f"{cfg.name}: max |out - f32 reference| = {err_all:.3e} over {got.size} values "
              f"(reference vs oracle {pin:.1e})")
        assert err_all <= tol(cfg.dtype)
        got = got[sel[:, 0], sel[:, 1], sel[:, 2]]
    err = float(np.abs(got - ref).max())
    print(f"{cfg.name}: max |out - oracle| = {err:.3e} over {ref.size} values")
    assert err <= tol(cfg.dtype)


CASES = [
    # dtype, B, Hq, Hkv, D, tree, prefix lens
    ("bf16", 1, 2, 1, 64, "c0", [0]),
    ("bf16", 3, 8, 2, 128, "c1", [1, 63, 129]),
    ("bf16", 2, 8, 1, 128, "c3", [64, 65]),
    ("bf16", 2, 16, 2, 64, "c2", [127, 300]),
    ("bf16", 1, 8, 8, 128, "c4", [5]),
    ("bf16", 1, 4, 1, 128, "chain8", [700]),
    ("bf16", 1, 16, 1, 64, "c3", [90]),           # 2064 query rows: 17 tiles, the last of 16 rows
    # 3 x 8 x 70 = 1680 work-groups: the 4-wave, two-row-block form of the kernel
    ("bf16", 3, 64, 8, 128, "c4", [3, 40, 64]),
    ("bf16", 3, 64, 8, 64, "c4", [0, 17, 65]),
    ("bf16", 2, 4, 4, 128, "one", [0, 3]),
    # 129 query rows per kv head with at least 256 (sequence, kv head) pairs: a 128-row tile of
    # the 4-wave kernel with the 129th row on the vector units (keys split over the waves)
    ("bf16", 2, 128, 128, 128, "c3", [64, 200]),
    ("bf16", 2, 128, 128, 128, "c3", [0, 1]),
    ("bf16", 2, 128, 128, 64, "c3", [63, 130]),
    ("bf16", 4, 192, 64, 128, "cart2x20", [5, 190, 0, 64]),   # 3 q heads x 43 nodes: (node 42, head 2)
    ("bf16", 1, 128, 128, 128, "cart16x15", [70]),      # 257 rows: only the first tile has one
    # 130 rows per kv head (two past the tile): one 144-row work-group of nine waves each
    ("bf16", 4, 128, 64, 64, "c1", [0, 1, 100, 63]),
    ("f32", 2, 4, 2, 64, "c1", [0, 77]),
    ("f32", 1, 2, 2, 128, "c0", [1]),
    ("f32", 1, 8, 1, 64, "c3", [200]),
    # the largest tree (4096 tokens, 64 tree tiles and mask words): 8192 rows per kv head
    ("bf16", 1, 2, 1, 128, "max4096", [100]),
    ("f32", 1, 2, 2, 64, "max4096", [5]),
]


def _choices(name):
    if name == "chain8":
        return cartesian_choices([1] * 8), 1, 8
    if name == "max4096":
        return cartesian_choices([63, 64]), 64, 2
    if name == "cart2x20":
        return cartesian_choices([2, 20]), 20, 2
    if name == "cart16x15":
        return cartesian_choices([16, 15]), 16, 2
    if name == "one":
        return [[0]], 1, 1
    return load_tree_choices(name), 10, 5


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-{c[5]}" for c in CASES])
def test_attention_edges(case):
    dtype, B, Hq, Hkv, D, tname, pls = case
    m = lib()
    choices, topk, K = _choices(tname)
    st = oracle.build_static(choices, topk, K)
    T = st["T"]
    cfg = custom(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, L=max(pls), seed=B * 13 + Hq)
    a = gen_attention_inputs(cfg, T, prefix_lens=pls, lcap=max(pls) + T + 37)
    # rows past L_b + T must never be read: poison them with NaN
    nan = np.float32("nan") if dtype == "f32" else np.uint16(0x7FC0)
    for b, L in enumerate(pls):
        a["k_cache"][b, :, L + T:] = nan
        a["v_cache"][b, :, L + T:] = nan
    say("attention edge", case)
    out = run_attn(m, a, mask_array(st), Hkv)
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], dtype, a["prefix_len"],
                                st["mask"], Hkv)
    got = as_f64(out, dtype)
    assert not np.isnan(got).any()
    err = float(np.abs(got - ref).max())
    print(f"{case}: max err {err:.3e}")
    assert err <= tol(dtype)


def test_attention_deterministic():
    m = lib()
    cfg = custom(dtype="bf16", B=1, Hq=32, Hkv=8, D=128, L=1500, seed=3)
    st = oracle.build_static(load_tree_choices("c2"), 10, 5)
    a = gen_attention_inputs(cfg, st["T"])
    say("attention determinism")
    o1 = run_attn(m, a, mask_array(st), 8)
    o2 = run_attn(m, a, mask_array(st), 8)
    assert np.array_equal(o1, o2)


def test_attention_extra_row_deterministic():
    m = lib()
    cfg = custom(dtype="bf16", B=2, Hq=128, Hkv=128, D=128, L=300, seed=5)
    st = oracle.build_static(load_tree_choices("c3"), 10, 5)
    a = gen_attention_inputs(cfg, st["T"])
    say("attention determinism, extra-row kernel")
    o1 = run_attn(m, a, mask_array(st), 128)
    o2 = run_attn(m, a, mask_array(st), 128)
    assert np.array_equal(o1, o2)


def _random_tree_exact(rng, n, topk=8, max_depth=6):
    """A random prefix-closed choice list of exactly n nodes (each new child takes its parent's
    next free rank)."""
    nodes, used = [()], {(): 0}
    while len(nodes) < n + 1:
        parent = nodes[int(rng.integers(len(nodes)))]
        if len(parent) >= max_depth or used[parent] >= topk:
            continue
        child = parent + (used[parent],)
        used[parent] += 1
        used[child] = 0
        nodes.append(child)
    return [list(t) for t in nodes[1:]]


# (G, T, B, Hkv, D): 128 * q + r rows per kv head, r in {1, 2}, with enough (sequence, kv head)
# pairs that the plan takes the extra rows; with two query tiles only the first r own one
XROW_CASES = [(1, 129, 2, 128, 128), (1, 129, 1, 256, 64), (1, 257, 1, 128, 128),
              (1, 258, 1, 128, 64), (2, 129, 1, 128, 128), (1, 129, 4, 64, 128)]


@pytest.mark.parametrize("i", range(len(XROW_CASES)))
def test_attention_extra_row_random(i):
    """Random trees and ragged prefixes on shapes the extra-row kernel takes; every output
    against the float32 device reference, itself pinned to the oracle on sampled units."""
    G, T, B, Hkv, D = XROW_CASES[i]
    rng = rng_for(1300 + i, 0)
    m = lib()
    st = oracle.build_static(_random_tree_exact(rng, T - 1), 8, 6)
    assert st["T"] == T
    pls = [int(x) for x in rng.choice([0, 1, 63, 64, 65, 200], size=B)]
    cfg = custom(dtype="bf16", B=B, Hq=G * Hkv, Hkv=Hkv, D=D, L=max(pls), seed=1300 + i)
    a = gen_attention_inputs(cfg, T, prefix_lens=pls, lcap=max(pls) + T + 5)
    nan = np.uint16(0x7FC0)
    for b, L in enumerate(pls):
        a["k_cache"][b, :, L + T:] = nan
        a["v_cache"][b, :, L + T:] = nan
    mask = mask_array(st)
    say("attention extra row", dict(G=G, T=T, B=B, Hkv=Hkv, D=D, pls=pls))
    out = as_f64(run_attn(m, a, mask, Hkv), "bf16")
    assert not np.isnan(out).any()
    sel = sample_units(B, G * Hkv, T, 200, 1300 + i)
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], "bf16", a["prefix_len"],
                                st["mask"], Hkv, sel=sel)
    ref = ref[sel[:, 0], sel[:, 1], sel[:, 2]]
    every = attention_all_f32(a["q"], a["k_cache"], a["v_cache"], a["prefix_len"], mask, Hkv)
    pin = float(np.abs(every[sel[:, 0], sel[:, 1], sel[:, 2]] - ref).max())
    assert pin <= 1e-4, pin
    assert float(np.abs(out[sel[:, 0], sel[:, 1], sel[:, 2]] - ref).max()) <= tol("bf16")
    err = float(np.abs(out - every).max())
    print(f"extra-row case {i}: max |out - f32 reference| = {err:.3e}, reference vs oracle {pin:.1e}")
    assert err <= tol("bf16")
