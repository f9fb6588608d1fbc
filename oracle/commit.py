"""Oracle: committing one verification step's accepted candidate (numpy).  Test infrastructure only.

Wiblog "Medusa multi-head speculative decoding", inference-flow section: acceptance walks from
the root until the first rejection or a leaf; the accepted prefix is then output, and the next
round starts from the hidden state of the last accepted token.  The verification logits already
hold that token's distribution, so the next round's first token needs no extra forward pass.

Readings where the pages are silent (plainest reading of the loop they describe):
  * the step emits the root followed by the accepted nodes of the best path: accept_length + 1
    tokens, padded with -1 up to the tree depth;
  * the cache keeps the accepted sequence in order: the K/V of the path's node at depth k moves
    from its tree row prefix_len + node to row prefix_len + k (the root already sits at
    prefix_len), and the prefix grows by accept_length + 1; every other cache row is unchanged;
  * the next step's root is next_token (the greedy token after the last accepted node) and its
    heads read the hidden state of the last accepted node.
"""

import numpy as np


def commit(static, best, accept_len, tokens, next_token, k_cache, v_cache, prefix_len,
           hidden=None):
    """static: oracle.build_static(...); best, accept_len, next_token, prefix_len: [B];
    tokens [B][T]; caches [B, Hkv, Lcap, D] (any dtype, returned as new arrays);
    hidden [B, T, Hd] or None.

    Returns dict(k_cache, v_cache, prefix_len, out_tokens [B, dmax+1], out_count [B],
    new_root [B], next_hidden [B, Hd] or None)."""
    B = len(best)
    T = static["T"]
    dmax = static["dmax"]
    kc, vc = k_cache.copy(), v_cache.copy()
    out_tokens = np.full((B, dmax + 1), -1, np.int32)
    out_count = np.zeros(B, np.int32)
    new_pl = np.array(prefix_len, np.int32).copy()
    new_root = np.array(next_token, np.int32).copy()
    next_hidden = None if hidden is None else np.zeros((B, hidden.shape[2]), hidden.dtype)
    for b in range(B):
        p, a, L = int(best[b]), int(accept_len[b]), int(prefix_len[b])
        path = static["paths"][p]
        assert 0 <= a <= static["path_len"][p] and 0 <= L and L + T <= k_cache.shape[2]
        for k in range(a + 1):
            out_tokens[b, k] = int(tokens[b][path[k]])
        out_count[b] = a + 1
        for k in range(1, a + 1):
            # destination row L + k takes the pre-commit row of node path[k]
            kc[b, :, L + k, :] = k_cache[b, :, L + path[k], :]
            vc[b, :, L + k, :] = v_cache[b, :, L + path[k], :]
        new_pl[b] = L + a + 1
        if hidden is not None:
            next_hidden[b] = hidden[b, path[a]]
    return dict(k_cache=kc, v_cache=vc, prefix_len=new_pl, out_tokens=out_tokens,
                out_count=out_count, new_root=new_root, next_hidden=next_hidden)
