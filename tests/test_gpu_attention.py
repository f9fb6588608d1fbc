"""GPU parity of tree_attention against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
from gpu_util import as_f64, dev, host, lib, mask_array, say, tol
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
    rng = rng_for(seed, 9)
    # every head of the first and the last sequence at a few nodes (the last sequence's units are
    # the ones the work plan runs last, cut into K/V splits), plus random rows
    sel = [(b, h, i) for b in {0, B - 1} for h in range(Hq) for i in {0, 1, T // 2, T - 1}]
    sel += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(n)]
    return np.array(sorted(set(sel)), np.int32)


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
    if sel is not None:
        got = got[sel[:, 0], sel[:, 1], sel[:, 2]]
        ref = ref[sel[:, 0], sel[:, 1], sel[:, 2]]
    else:
        assert not np.isnan(got).any()
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
    ("f32", 2, 4, 2, 64, "c1", [0, 77]),
    ("f32", 1, 2, 2, 128, "c0", [1]),
    ("f32", 1, 8, 1, 64, "c3", [200]),
]


def _choices(name):
    if name == "chain8":
        return cartesian_choices([1] * 8), 1, 8
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
