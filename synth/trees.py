"""Tree choice lists (the `medusa_choices` input): one rank tuple per non-root node.

A node (r1, ..., rd) is the candidate made of head 1's rank-r1 token, then head 2's rank-r2
token, ..., head d's rank-rd token.  The pages give two explicit trees: top-2 x top-3
(Wiblog page, tree-attention section; Ultralytics page, tree-attention section) and the full
K=3, k=10 product of up to 1000 candidates (jisaku page, how-it-works).  For the 64/128-node
sparse trees they say only that the tree is built from the most accurate combinations
(Ultralytics page, tree-attention section), so a synthetic rule stands in:

  * rank-r accuracy of every head s(r) = 0.6 * (r+1)^(-gamma), gamma = 2.35, fitted so that
    s(0) = 0.60 and s(0)+...+s(4) = 0.80 (top-1 about 60 %, top-5 above 80 %: Wiblog page,
    heads section);
  * node score d*ln(0.6) - gamma*ln(prod(r_i+1)), fp64 from the integers;
  * keep the N best, ties broken by depth then rank tuple ascending.  Every child scores below
    its parent, so the selection is prefix-closed.

The lists are written once by `python -m synth.trees` into synth/trees/*.json.
"""

import itertools
import json
import math
import os

GAMMA = 2.35
HERE = os.path.join(os.path.dirname(__file__), "trees")

SPARSE = {"c1": (64, 4), "c2": (64, 5), "c3": (128, 3)}


def _score(t):
    p = 1
    for r in t:
        p *= r + 1
    return len(t) * math.log(0.6) - GAMMA * math.log(p)


def sparse_tree_choices(n_nodes, max_depth, k=10):
    cands = [t for d in range(1, max_depth + 1) for t in itertools.product(range(k), repeat=d)]
    cands.sort(key=lambda t: (-_score(t), len(t), t))
    return [list(t) for t in cands[:n_nodes]]


def cartesian_choices(ks):
    """All prefixes of the product range(ks[0]) x range(ks[1]) x ... (a dense tree)."""
    out = []
    for d in range(1, len(ks) + 1):
        out += [list(t) for t in itertools.product(*[range(k) for k in ks[:d]])]
    return out


def all_trees():
    trees = {"c0": cartesian_choices([2, 3]), "c4": cartesian_choices([10, 10, 10])}
    for name, (n, d) in SPARSE.items():
        trees[name] = sparse_tree_choices(n, d)
    return trees


def load_tree_choices(name):
    with open(os.path.join(HERE, name + ".json")) as f:
        return json.load(f)["choices"]


def write_all():
    os.makedirs(HERE, exist_ok=True)
    for name, ch in all_trees().items():
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump({"name": name, "n_nodes": len(ch), "choices": ch}, f, separators=(",", ":"))


if __name__ == "__main__":
    write_all()
