"""Oracle: the N-node candidate tree of largest expected accept length.  Test infrastructure only.

Ultralytics "Medusa Heads", tree-attention section: a sparse tree built from the most accurate
combinations of head candidates speeds decoding up more than a dense tree several times its
size.  Wiblog "Medusa multi-head speculative decoding", heads section: a head's top-1 candidate
is right about 60 % of the time and its top-5 more than 80 %.

Reading where the pages stop (they give no formula):
  * head k's rank-r candidate is the right token with probability acc[k][r], independently
    across heads, and at most one candidate of a head is right;
  * the accept length is the depth of the deepest tree node whose rank tuple is the right one,
    so P(accept length >= d) is the sum over depth-d nodes of P(node right), and
        E[accept length] = sum over tree nodes of prod_k acc[k][r_k];
  * a node is never more likely than its parent, so the N most likely nodes (ties: depth, then
    rank tuple) form a tree, and no other N-node tree has a larger expectation.
Node probabilities are the product taken in depth order in fp64, so equal products are exact
ties; the expectation is summed in node order (depth, then rank tuple).
"""

import itertools


def node_prob(acc, t):
    p = 1.0
    for k, r in enumerate(t):
        p = p * float(acc[k][r])
    return p


def all_nodes(K, topk):
    return [t for d in range(1, K + 1) for t in itertools.product(range(topk), repeat=d)]


def sparse_tree(acc, N):
    """acc [K][topk] (nested lists or array).  Returns (choices in node order, expectation)."""
    K, topk = len(acc), len(acc[0])
    nodes = all_nodes(K, topk)
    assert 1 <= N <= len(nodes)
    nodes.sort(key=lambda t: (-node_prob(acc, t), len(t), t))
    sel = sorted(nodes[:N], key=lambda t: (len(t), t))
    exp_len = 0.0
    for t in sel:
        exp_len += node_prob(acc, t)
    return [list(t) for t in sel], exp_len


def expected_accept_length(acc, choices):
    """The objective for any choice list, summed in node order."""
    total = 0.0
    for t in sorted((tuple(c) for c in choices), key=lambda t: (len(t), t)):
        total += node_prob(acc, t)
    return total
