"""Pins for the oracle's typical acceptance.

Closed forms of p > min(eps, delta*exp(-H)) on rows whose probabilities are set exactly through
log-probabilities, the greedy limit at temperature 0 (Wiblog page, typical-acceptance section;
Ultralytics page, tree-attention section), the falling threshold as temperature rises (Wiblog
page, acceptance-rate section), and the longest-prefix walk checked by an independent
leaf-to-root brute force.  The rows are built so that a max in place of the min, log2 in place of
ln, a flipped entropy sign, or a child judged by its own row instead of its parent's fails.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.accept import row_threshold
from synth.gen import rng_for
from synth.trees import cartesian_choices, load_tree_choices

EPS, DELTA = 0.09, 0.3


def _tree_with_root_children(n_children):
    return oracle.build_static([[r] for r in range(n_children)], n_children, 1)


def _logits_from_probs(p, V):
    """One row whose softmax is p (zero entries get -inf)."""
    row = np.full(V, -np.inf)
    row[:len(p)] = np.log(p)
    return row


def _run_single_row(row, child_tokens, temperature=1.0):
    st = _tree_with_root_children(len(child_tokens))
    T = st["T"]
    V = row.shape[0]
    logits = np.zeros((1, T, V), np.float32)
    logits[0, 0] = row
    tokens = [[0] + list(child_tokens)]
    return oracle.typical_accept(logits, "f32", tokens, st, temperature, EPS, DELTA)


def test_defaults_from_the_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "accept_params.json")))
    assert g["default"] == {"posterior_threshold": EPS, "posterior_alpha": DELTA}
    assert math.isclose(math.sqrt(g["default"]["posterior_threshold"]),
                        g["default"]["posterior_alpha"])


def test_hard_threshold_binds_on_a_confident_row():
    # p = [0.8, 0.1, 0.06, 0.04]: H = 0.706 nats, delta*e^-H = 0.148 > eps -> thr = 0.09
    p = [0.8, 0.1, 0.06, 0.04]
    res = _run_single_row(_logits_from_probs(p, 8), [0, 1, 2, 3])
    assert res["accepted"][0, 1:].tolist() == [True, True, False, False]
    _, H, thr = row_threshold(_logits_from_probs(p, 8).astype(np.float32).astype(np.float64),
                              EPS, DELTA)
    assert abs(H - 0.7063) < 1e-3 and thr == EPS


def test_entropy_threshold_binds_on_a_flat_row():
    # 100 tokens share 0.998, one token has 0.002 = 0.2/100: H ~ ln 100, thr ~ 0.3/100.
    n = 100
    p = [0.998 / n] * n + [0.002]
    res = _run_single_row(_logits_from_probs(p, 128), [0, 57, n])
    assert res["accepted"][0, 1:].tolist() == [True, True, False]
    _, H, thr = row_threshold(_logits_from_probs(p, 128), EPS, DELTA)
    assert abs(H - math.log(n)) < 0.02
    assert abs(thr - DELTA * math.exp(-H)) < 1e-15 and thr < EPS


@pytest.mark.parametrize("n,binding", [(3, "eps"), (4, "entropy")])
def test_switch_point_between_the_two_thresholds(n, binding):
    # uniform over n: H = ln n; the entropy term takes over above H* = ln(delta/eps) = 1.204
    _, H, thr = row_threshold(_logits_from_probs([1.0 / n] * n, 16), EPS, DELTA)
    assert abs(H - math.log(n)) < 1e-12
    if binding == "eps":
        assert thr == EPS
    else:
        assert abs(thr - DELTA / n) < 1e-15
    assert (math.log(n) > math.log(DELTA / EPS)) == (binding == "entropy")


def test_uniform_row_accepts_every_token():
    V = 1000
    res = _run_single_row(np.zeros(V), [0, 999, 500])
    assert res["accepted"][0, 1:].all()     # p = 1/V > delta/V because delta < 1


def test_two_point_row_accepts_both():
    res = _run_single_row(_logits_from_probs([0.5, 0.5], 10), [0, 1, 2])
    assert res["accepted"][0, 1:].tolist() == [True, True, False]


def test_temperature_zero_is_greedy_with_lowest_id_on_ties():
    row = np.array([1.0, 3.0, 3.0, 2.0, -1.0])
    res = _run_single_row(row, [1, 2, 3], temperature=0)
    assert res["accepted"][0, 1:].tolist() == [True, False, False]


def test_small_temperature_equals_greedy():
    rng = rng_for(31, 0)
    choices = load_tree_choices("c1")
    st = oracle.build_static(choices, 10, 4)
    T, V = st["T"], 64
    for trial in range(5):
        logits = (rng.standard_normal((1, T, V)) * 2).astype(np.float32)
        tokens = [[int(x) for x in rng.integers(0, V, T)]]
        # make half of the children equal to their parent row's argmax
        for c in range(1, T):
            if rng.random() < 0.5:
                tokens[0][c] = int(np.argmax(logits[0, st["parent"][c]]))
        gaps = np.sort(logits[0], axis=1)
        min_gap = float((gaps[:, -1] - gaps[:, -2]).min())
        g = oracle.typical_accept(logits, "f32", tokens, st, 0)
        s = oracle.typical_accept(logits, "f32", tokens, st, min_gap / 50)
        assert np.array_equal(g["accepted"], s["accepted"])
        assert g["best_candidate"].tolist() == s["best_candidate"].tolist()
        assert g["accept_length"].tolist() == s["accept_length"].tolist()


def test_power_of_two_scaling_is_invisible():
    rng = rng_for(32, 0)
    st = oracle.build_static(load_tree_choices("c0"), 3, 2)
    logits = (rng.standard_normal((2, st["T"], 50)) * 2).astype(np.float32)
    tokens = rng.integers(0, 50, (2, st["T"])).tolist()
    a = oracle.typical_accept(logits, "f32", tokens, st, 0.7)
    b = oracle.typical_accept(logits * 2, "f32", tokens, st, 1.4)
    assert np.array_equal(a["accepted"], b["accepted"])
    np.testing.assert_allclose(a["threshold"], b["threshold"], rtol=1e-14)


def test_threshold_falls_as_temperature_rises():
    rng = rng_for(33, 0)
    row = rng.standard_normal(3000) * 2
    thr = [row_threshold(row / t, EPS, DELTA)[2] for t in (0.3, 0.5, 0.7, 1.0, 1.5, 3.0)]
    assert all(a >= b for a, b in zip(thr, thr[1:]))
    assert thr[-1] < thr[0]


def _brute_best(st, accepted):
    """Independent walk: for each leaf go up to the root, then count accepted nodes from the top."""
    leaves = [i for i in range(st["T"]) if not st["children"][i]]
    leaves.sort(key=lambda i: st["nodes"][i])
    best, blen = None, -1
    for p, leaf in enumerate(leaves):
        chain = []
        j = leaf
        while j != 0:
            chain.append(j)
            j = st["parent"][j]
        chain.reverse()
        n = 0
        for node in chain:
            if not accepted[node]:
                break
            n += 1
        if n > blen:
            best, blen = p, n
    return best, blen


@pytest.mark.parametrize("tree", ["c0", "c1", "c2", "c3"])
def test_longest_accepted_prefix_by_brute_force(tree):
    rng = rng_for(34, 0)
    st = oracle.build_static(load_tree_choices(tree), 10, 5)
    T, V = st["T"], 40
    for trial in range(10):
        # at T = 0 a child is accepted iff its token is its parent row's argmax: plant decisions
        logits = rng.standard_normal((1, T, V)).astype(np.float32)
        want = rng.random(T) < 0.6
        tokens = [0] * T
        for c in range(1, T):
            am = int(np.argmax(logits[0, st["parent"][c]]))
            tokens[c] = am if want[c] else (am + 1 + int(rng.integers(0, V - 1))) % V
        res = oracle.typical_accept(logits, "f32", [tokens], st, 0)
        dec = res["accepted"][0]
        assert dec[1:].tolist() == want[1:].tolist()
        best, blen = _brute_best(st, dec)
        assert res["best_candidate"][0] == best and res["accept_length"][0] == blen
        last = st["paths"][best][blen]
        assert res["next_token"][0] == int(np.argmax(logits[0, last]))
        assert 0 <= blen <= st["path_len"][best]


def test_child_is_judged_by_its_parents_row():
    st = oracle.build_static(cartesian_choices([1, 1]), 1, 2)   # root -> a -> b
    V = 8
    logits = np.zeros((1, 3, V), np.float32)
    logits[0, 0, 5] = 10.0       # root row favours token 5 (node a)
    logits[0, 1, 6] = 10.0       # a's row favours token 6 (node b)
    logits[0, 2, 1] = 10.0       # b's row (a leaf) only matters for next_token
    res = oracle.typical_accept(logits, "f32", [[0, 5, 6]], st, 0)
    assert res["accept_length"][0] == 2 and res["next_token"][0] == 1
    res = oracle.typical_accept(logits, "f32", [[0, 6, 5]], st, 0)
    assert res["accept_length"][0] == 0 and res["next_token"][0] == 5


def test_first_token_always_yields_progress():
    rng = rng_for(35, 0)
    st = oracle.build_static(load_tree_choices("c0"), 3, 2)
    logits = (rng.standard_normal((3, st["T"], 20)) * 2).astype(np.float32)
    tokens = rng.integers(0, 20, (3, st["T"])).tolist()
    for t in (0, 0.7):
        res = oracle.typical_accept(logits, "f32", tokens, st, t)
        assert (res["accept_length"] + 1 >= 1).all()
        assert (res["accept_length"] <= st["dmax"]).all()


def test_equality_rejects():
    # uniform over 4: p = 1/4 exactly; eps = 1/4 and a large delta make thr = 1/4 exactly
    st = _tree_with_root_children(2)
    logits = np.zeros((1, st["T"], 4), np.float32)
    res = oracle.typical_accept(logits, "f32", [[0, 1, 2]], st, 1.0, eps=0.25, delta=10.0)
    assert res["threshold"][0, 0] == 0.25
    assert not res["accepted"][0, 1:].any()


# ---- nucleus mode of evaluate_posterior (reading: candidate in the top_p nucleus of p) ----

def _nucleus_single_row(row, child_tokens, top_p, temperature=1.0):
    st = _tree_with_root_children(len(child_tokens))
    T = st["T"]
    logits = np.zeros((1, T, len(row)), np.float64)
    logits[0, 0] = row
    tokens = [[0] + list(child_tokens)]
    return oracle.evaluate_posterior(logits, "f64", tokens, st, temperature, top_p=top_p,
                                     sampling="nucleus")


def test_nucleus_hand_worked_row():
    # p = [0.5, 0.25, 0.125, 0.125, 0]: the mass strictly above each token is 0, 0.5, 0.75,
    # 0.75 (tokens 2 and 3 tie) and 1 (the -inf token)
    row = _logits_from_probs([0.5, 0.25, 0.125, 0.125], 5)
    for top_p, want in [(0.49, [1, 0, 0, 0, 0]), (0.51, [1, 1, 0, 0, 0]), (0.74, [1, 1, 0, 0, 0]),
                        (0.76, [1, 1, 1, 1, 0]), (1.0, [1, 1, 1, 1, 0])]:
        res = _nucleus_single_row(row, [0, 1, 2, 3, 4], top_p)
        assert res["accepted"][0, 1:].astype(int).tolist() == want, top_p
    res = _nucleus_single_row(row, [0, 1, 2, 3, 4], 0.6)
    assert np.isinf(res["margin"][0, 1]) and res["margin"][0, 1] > 0      # nothing above the max
    assert abs(res["margin"][0, 2] - (math.log(0.6) - math.log(0.5))) < 1e-12
    assert abs(res["margin"][0, 3] - (math.log(0.6) - math.log(0.75))) < 1e-12


def test_nucleus_ties_at_the_cut_go_in_together():
    # p = [0.4, 0.3, 0.3], top_p = 0.5: both tied tokens have 0.4 above them, so both are in
    # the nucleus (a sorted prefix would keep only one, depending on the sort)
    row = _logits_from_probs([0.4, 0.3, 0.3], 3)
    res = _nucleus_single_row(row, [2, 1, 0], 0.5)
    assert res["accepted"][0, 1:].tolist() == [True, True, True]
    res = _nucleus_single_row(row, [2, 1, 0], 0.4)
    assert res["accepted"][0, 1:].tolist() == [False, False, True]


def test_nucleus_matches_a_sorted_prefix_without_ties():
    # brute force: sort descending, keep the shortest prefix whose mass reaches top_p; on rows
    # without ties a token is in it iff the mass strictly above it is below top_p
    rng = rng_for(61, 0)
    for trial in range(40):
        V = int(rng.integers(2, 60))
        row = rng.standard_normal(V) * 2.0
        temp = float(rng.uniform(0.3, 2.0))
        top_p = float(rng.uniform(0.05, 0.99))
        z = row / temp
        p = np.exp(z - z.max())
        p /= p.sum()
        order = np.argsort(-p, kind="stable")
        csum = np.cumsum(p[order])
        j = int(np.searchsorted(csum, top_p)) + 1          # first prefix with mass >= top_p
        inside = set(order[:j].tolist())
        if any(abs(c - top_p) < 1e-9 for c in csum):
            continue
        kids = [int(x) for x in rng.choice(V, size=min(V, 6), replace=False)]
        res = _nucleus_single_row(row, kids, top_p, temp)
        assert res["accepted"][0, 1:].tolist() == [k in inside for k in kids], trial


def test_nucleus_limits():
    rng = rng_for(62, 0)
    st = oracle.build_static(load_tree_choices("c1"), 10, 4)
    V = 500
    logits = rng.standard_normal((2, st["T"], V)).astype(np.float32) * 2
    tokens = rng.integers(0, V, (2, st["T"])).tolist()
    for b in range(2):
        for c in range(1, st["T"]):             # some children are their parent row's argmax
            if c % 3 == 0:
                tokens[b][c] = int(np.argmax(logits[b, st["parent"][c]]))
    greedy = oracle.typical_accept(logits, "f32", tokens, st, 0.0)
    # a nucleus smaller than any probability holds only the maximum: greedy decisions
    tiny = oracle.evaluate_posterior(logits, "f32", tokens, st, 0.7, top_p=1e-9,
                                     sampling="nucleus")
    assert np.array_equal(tiny["accepted"], greedy["accepted"])
    assert tiny["accept_length"].tolist() == greedy["accept_length"].tolist()
    # the whole distribution: every candidate with a finite logit is in it
    full = oracle.evaluate_posterior(logits, "f32", tokens, st, 0.7, top_p=1.0,
                                     sampling="nucleus")
    assert full["accepted"].all()
    assert full["accept_length"].tolist() == [max(st["path_len"])] * 2
    # temperature 0 is greedy in nucleus mode too, and the fast flag changes nothing
    g2 = oracle.evaluate_posterior(logits, "f32", tokens, st, 0.0, top_p=0.5, sampling="nucleus",
                                   fast=True)
    assert np.array_equal(g2["accepted"], greedy["accepted"])
    typ = oracle.evaluate_posterior(logits, "f32", tokens, st, 0.7, sampling="typical", fast=True)
    ref = oracle.typical_accept(logits, "f32", tokens, st, 0.7)
    assert np.array_equal(typ["accepted"], ref["accepted"])


def test_nucleus_widens_with_temperature():
    # a hotter distribution is flatter, so the mass above a low-ranked token grows and fewer
    # low-ranked candidates stay in a fixed-mass nucleus; at a very high temperature the mass
    # above the rank-r token tends to r / V
    row = np.linspace(3.0, -3.0, 50)
    cold = _nucleus_single_row(row, list(range(50)), 0.9, temperature=0.5)
    hot = _nucleus_single_row(row, list(range(50)), 0.9, temperature=5.0)
    assert cold["accepted"][0, 1:].sum() < hot["accepted"][0, 1:].sum()
    vhot = _nucleus_single_row(row, list(range(50)), 0.3, temperature=1e6)
    assert vhot["accepted"][0, 1:].astype(int).tolist() == [1] * 15 + [0] * 35
