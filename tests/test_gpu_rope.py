"""GPU parity of tree_attention_rope against the oracle, through the C ABI.

Outputs within the attention tolerance.  The rotated key rows written back into the cache equal
the oracle's (rounded from the exact value) except where fp32 arithmetic moves the value across a
bf16 rounding boundary: one bf16 step, or ~1e-6 absolute where the rotation cancels to a tiny
value; such elements must stay rare.  Rows outside the tree, and q, are untouched."""

import numpy as np
import pytest

import oracle
from gpu_util import as_f64, attention_all_f32, dev, host, lib, mask_array, say, tol
from synth import get_config
from synth.configs import custom
from synth.gen import gen_attention_inputs
from synth.trees import load_tree_choices

pytestmark = pytest.mark.gpu


def run_rope(m, a, mask, Hkv, pos, base):
    import torch
    q, kc, vc = dev(a["q"]), dev(a["k_cache"]), dev(a["v_cache"])
    B, Hq, T, D = a["q"].shape
    L = int(np.max(a["prefix_len"]))
    ws = m.workspace(m.tree_attention_rope_workspace(B, Hq, Hkv, T, D, L))
    out = torch.empty_like(q)
    q0 = q.clone()
    m.tree_attention_rope(q, kc, vc, dev(a["prefix_len"]), L, dev(mask.view(np.int64)), dev(pos), out, ws,
                          rope_base=base)
    torch.cuda.synchronize()
    assert torch.equal(q, q0), "q must not change"
    return host(out), host(kc)


def check_keys(got, ref, dtype, T, pls):
    for b, L in enumerate(pls):
        g, r = got[b], ref[b]
        if dtype == "bf16":
            # one bf16 step of the result, plus fp32 rounding of unit-scale inputs where the
            # rotation cancels to a tiny value
            gf, rf = as_f64(g, dtype), as_f64(r, dtype)
            err = np.abs(gf - rf)
            assert (err <= np.abs(rf) * 2.0 ** -7 + 1e-6).all(), float(err.max())
            assert (g != r).mean() <= 2e-3, (g != r).mean()
        else:
            np.testing.assert_allclose(g, r, rtol=2e-6, atol=2e-6)
        assert np.array_equal(g[:, :L], r[:, :L]) and np.array_equal(g[:, L + T:], r[:, L + T:])


@pytest.mark.parametrize("ci,base", [(0, 10000.0), (1, 10000.0), (2, 500000.0), (3, 10000.0),
                                     (4, 500000.0)])
def test_rope_attention_full_size(ci, base):
    cfg = get_config(ci)
    m = lib()
    st = oracle.build_static(load_tree_choices(f"c{ci}"), cfg.topk, cfg.K)
    T = st["T"]
    a = gen_attention_inputs(cfg, T)
    pos = np.array([[int(a["prefix_len"][b]) + d for d in st["depth"]] for b in range(cfg.B)],
                   np.int32)
    say("rope attention full size", cfg.name, base)
    out, kc = run_rope(m, a, mask_array(st), cfg.Hkv, pos, base)
    qr, kr = oracle.rotate_tree(a["q"], a["k_cache"], cfg.dtype, a["prefix_len"], pos, base)
    check_keys(kc, kr, cfg.dtype, T, a["prefix_len"])
    sel = None
    if ci >= 3:
        rng = np.random.default_rng(ci)
        sel = np.stack([rng.integers(0, cfg.B, 300), rng.integers(0, cfg.Hq, 300),
                        rng.integers(0, T, 300)], 1).astype(np.int32)
    ref = oracle.tree_attention(qr, kr, a["v_cache"], cfg.dtype, a["prefix_len"], st["mask"],
                                cfg.Hkv, sel=sel)
    got = as_f64(out, cfg.dtype)
    assert not np.isnan(got).any()
    if sel is not None:
        ref = ref[sel[:, 0], sel[:, 1], sel[:, 2]]
        # every output against a float32 device reference over the oracle's rotated q and keys,
        # pinned to the oracle on the sampled units
        every = attention_all_f32(qr, kr, a["v_cache"], a["prefix_len"], mask_array(st), cfg.Hkv)
        pin = float(np.abs(every[sel[:, 0], sel[:, 1], sel[:, 2]] - ref).max())
        assert pin <= 1e-4, pin
        err_all = float(np.abs(got - every).max())
        print(f"{cfg.name}: max |out - f32 reference| = {err_all:.3e} over {got.size} values")
        assert err_all <= tol(cfg.dtype)
        got = got[sel[:, 0], sel[:, 1], sel[:, 2]]
    err = float(np.abs(got - ref).max())
    print(f"{cfg.name}: max |out - oracle| = {err:.3e}")
    assert err <= tol(cfg.dtype)


@pytest.mark.parametrize("dtype,D,B,Hq,Hkv,tree,pls,posmode", [
    ("bf16", 128, 2, 8, 2, "c1", [0, 300], "depth"),
    ("bf16", 64, 3, 4, 4, "c0", [5, 77, 1], "far"),        # positions near 100000
    ("f32", 64, 2, 4, 2, "c3", [40, 0], "depth"),
    ("f32", 128, 1, 2, 1, "c2", [123], "far"),
    ("f32", 128, 1, 40, 8, "c1", [9], "depth"),        # 8 key rows per node: one full chunk
    ("bf16", 64, 2, 32, 8, "c1", [3, 64], "far"),      # 8 rows per instruction, half a chunk
    ("bf16", 128, 2, 12, 12, "c0", [17, 250], "depth"),  # 12 rows: a full chunk and a ragged one
    ("f32", 64, 1, 40, 20, "c3", [31], "far"),         # 20 rows: chunks of 16 and 4
])
def test_rope_attention_edges(dtype, D, B, Hq, Hkv, tree, pls, posmode):
    m = lib()
    st = oracle.build_static(load_tree_choices(tree), 10, 5)
    T = st["T"]
    cfg = custom(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, L=max(pls), seed=B * 7 + D)
    a = gen_attention_inputs(cfg, T, prefix_lens=pls, lcap=max(pls) + T + 9)
    if posmode == "depth":
        pos = np.array([[pls[b] + d for d in st["depth"]] for b in range(B)], np.int32)
    else:
        pos = np.array([[99000 + 37 * b + d for d in st["depth"]] for b in range(B)], np.int32)
    say("rope attention edge", dtype, D, tree, pls, posmode)
    out, kc = run_rope(m, a, mask_array(st), Hkv, pos, 10000.0)
    qr, kr = oracle.rotate_tree(a["q"], a["k_cache"], dtype, a["prefix_len"], pos)
    check_keys(kc, kr, dtype, T, pls)
    ref = oracle.tree_attention(qr, kr, a["v_cache"], dtype, a["prefix_len"], st["mask"], Hkv)
    err = float(np.abs(as_f64(out, dtype) - ref).max())
    print(f"edge {dtype} D{D} {tree}: max err {err:.3e}")
    assert err <= tol(dtype)


@pytest.mark.parametrize("G,T,B,Hkv,D,base", [(1, 129, 2, 128, 128, 10000.0),
                                              (2, 129, 1, 128, 64, 500000.0)])
def test_rope_attention_extra_row(G, T, B, Hkv, D, base):
    """Rotary attention on shapes the extra-row kernel takes (random trees, ragged prefixes):
    the extra row's query is rotated in registers like the others.  Every output against the
    float32 device reference over the oracle's rotated q and keys, pinned to the oracle."""
    from test_gpu_attention import _random_tree_exact
    from synth.gen import rng_for
    m = lib()
    rng = rng_for(1400 + G * 7 + D, 0)
    st = oracle.build_static(_random_tree_exact(rng, T - 1), 8, 6)
    pls = [int(x) for x in rng.choice([0, 1, 63, 64, 65, 200], size=B)]
    cfg = custom(dtype="bf16", B=B, Hq=G * Hkv, Hkv=Hkv, D=D, L=max(pls), seed=1400 + D)
    a = gen_attention_inputs(cfg, T, prefix_lens=pls)
    pos = np.array([[pls[b] + d for d in st["depth"]] for b in range(B)], np.int32)
    say("rope attention, extra row", dict(G=G, T=T, B=B, Hkv=Hkv, D=D, pls=pls))
    out, kc = run_rope(m, a, mask_array(st), Hkv, pos, base)
    qr, kr = oracle.rotate_tree(a["q"], a["k_cache"], "bf16", a["prefix_len"], pos, base)
    check_keys(kc, kr, "bf16", T, a["prefix_len"])
    rs = np.random.default_rng(1400 + G)
    sel = np.stack([rs.integers(0, B, 300), rs.integers(0, G * Hkv, 300),
                    np.full(300, T - 1)], 1).astype(np.int32)   # the last node: the extra row
    ref = oracle.tree_attention(qr, kr, a["v_cache"], "bf16", a["prefix_len"], st["mask"], Hkv,
                                sel=sel)[sel[:, 0], sel[:, 1], sel[:, 2]]
    every = attention_all_f32(qr, kr, a["v_cache"], a["prefix_len"], mask_array(st), Hkv)
    pin = float(np.abs(every[sel[:, 0], sel[:, 1], sel[:, 2]] - ref).max())
    assert pin <= 1e-4, pin
    got = as_f64(out, "bf16")
    assert not np.isnan(got).any()
    assert float(np.abs(got[sel[:, 0], sel[:, 1], sel[:, 2]] - ref).max()) <= tol("bf16")
    err = float(np.abs(got - every).max())
    print(f"rope extra row G={G} D={D}: max |out - f32 reference| = {err:.3e}")
    assert err <= tol("bf16")
