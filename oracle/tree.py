"""Oracle: the fixed candidate tree (pure Python, integers only).  Test infrastructure only.

Wiblog "Medusa multi-head speculative decoding", tree-attention section: every head's top-k
candidates combine into a tree; a node is a token, a root-to-leaf path is a candidate sequence
(2 candidates from head 1 x 3 from head 2 give 6 paths of depth 2).  Each token may attend only
to the tokens on its own prefix path, never across paths, and position ids follow the path.  The
tree is fixed, so the mask is precomputed and cached.  Ultralytics "Medusa Heads",
tree-attention section: the mask lets each token see only its ancestors.  cnnetsun page,
configuration section: `medusa_choices` configures the tree.

Readings where the pages are silent:
  * a choice is a rank tuple (r1..rd); node (r1..rd) carries head d's rank-rd token, so head d
    fills depth d; the root (depth 0) is the last accepted token, passed in;
  * node order: root first, then by (depth, rank tuple) ascending, so a parent precedes its
    children;
  * a node sees itself and its ancestors (the root included); the prefix is fully visible;
  * position id = prefix_len + depth;
  * paths: one per leaf, leaves in ascending rank-tuple order.
"""


class TreeError(ValueError):
    pass


def canonical(choices, topk, K):
    """Validate a choice list and return its rank tuples in node order (root excluded)."""
    seen = set()
    for c in choices:
        t = tuple(int(r) for r in c)
        if len(t) == 0:
            raise TreeError("empty choice")
        if len(t) > K:
            raise TreeError(f"depth {len(t)} exceeds head count {K}")
        if any(r < 0 or r >= topk for r in t):
            raise TreeError(f"rank out of range in {t}")
        if t in seen:
            raise TreeError(f"duplicate choice {t}")
        seen.add(t)
    for t in seen:
        if len(t) > 1 and t[:-1] not in seen:
            raise TreeError(f"choice {t} has no parent {t[:-1]}")
    return sorted(seen, key=lambda t: (len(t), t))


def build_static(choices, topk, K):
    """The per-tree arrays: everything that does not depend on the step's tokens."""
    nodes = [()] + canonical(choices, topk, K)
    T = len(nodes)
    index = {t: i for i, t in enumerate(nodes)}
    depth = [len(t) for t in nodes]
    parent = [-1] + [index[t[:-1]] for t in nodes[1:]]
    W = (T + 63) // 64
    mask = [[0] * W for _ in range(T)]
    for i, ti in enumerate(nodes):
        for j, tj in enumerate(nodes):
            if ti[:len(tj)] == tj:          # j's rank tuple is a prefix of i's (or equal)
                mask[i][j // 64] |= 1 << (j % 64)
    children = [[] for _ in range(T)]
    for i in range(1, T):
        children[parent[i]].append(i)
    leaves = sorted((t for t in nodes[1:] if not children[index[t]]))
    dmax = max(depth)
    paths = []
    for leaf in leaves:
        row = [index[leaf[:d]] for d in range(len(leaf) + 1)]
        paths.append(row + [-1] * (dmax + 1 - len(row)))
    return dict(T=T, W=W, nodes=nodes, depth=depth, parent=parent, mask=mask,
                children=children, paths=paths, path_len=[len(l) for l in leaves], dmax=dmax,
                rank=[t[-1] if t else -1 for t in nodes])


def gather(static, topk_ids, root_tokens, prefix_len):
    """tokens[b][i] and position ids for one step.  topk_ids [B][K][k]."""
    B = len(root_tokens)
    tokens, pos = [], []
    for b in range(B):
        tb, pb = [], []
        for i, t in enumerate(static["nodes"]):
            d = len(t)
            tb.append(int(root_tokens[b]) if d == 0 else int(topk_ids[b][d - 1][t[-1]]))
            pb.append(int(prefix_len[b]) + d)
        tokens.append(tb)
        pos.append(pb)
    return tokens, pos


def mask_words_u64(static):
    """The mask as a [T][W] list of unsigned 64-bit words (bit j%64 of word j//64)."""
    return [list(r) for r in static["mask"]]
