"""Oracle: typical acceptance over the verification logits (fp64, numpy).  Test infrastructure.

Wiblog "Medusa multi-head speculative decoding":
  * typical-acceptance section: a candidate is kept when its probability under the original
    model exceeds a threshold taken as the minimum of a hard threshold and an entropy-dependent
    one; the first token is always taken greedily, so every step yields at least one token; the
    output is the longest prefix that passes; at temperature 0 this reduces to greedy decoding;
  * inference-flow section: walk from the root, accept while the test passes, stop at the first
    rejection or a leaf;
  * acceptance-rate section: higher temperature flattens p, raises the entropy and lowers the
    threshold.
Ultralytics "Medusa Heads", tree-attention section: under greedy decoding a candidate is accepted
when it equals the model's best choice.  cnnetsun page, architecture section: defaults
posterior_threshold = 0.09 and posterior_alpha = 0.3; the call returns
(best_candidate, accept_length).

The rule written out (the plainest reading consistent with all of the above):
  z = logits / T,  p = softmax(z),  H = -sum p ln p,  thr = min(eps, delta * exp(-H)),
  child c of node n accepted  iff  p_n(tok(c)) > thr_n            (T > 0)
                              iff  tok(c) == argmax_v logits_n[v]  (T = 0, lowest id on ties).
Row n of the logits is the distribution after node n, so child c is judged by row parent(c).
accept_length counts accepted nodes below the root along the best path (the root token itself
is the greedy first token and is not tested); best_candidate is the lowest path index with the
largest count; next_token is the argmax of the row of the last accepted node on that path.
"""

import numpy as np

from . import bf16


def _row_f64(logits, dtype, b, n):
    return bf16.to_f64(logits[b, n], dtype)


def _argmax_lowest(x):
    m = x.max()
    return int(np.flatnonzero(x == m)[0])


def row_threshold(z_row, eps, delta):
    """p, H and the typical-acceptance threshold of one row of temperature-scaled logits."""
    m = z_row.max()
    e = np.exp(z_row - m)
    p = e / e.sum()
    nz = p > 0
    H = -np.sum(p[nz] * np.log(p[nz]))
    thr = min(eps, delta * np.exp(-H))
    return p, H, thr


def scan_paths(static, accepted_b):
    """Longest run of accepted nodes below the root along each root-to-leaf path.  Returns
    (best path = lowest index among the longest, its accept length, last accepted node)."""
    paths, path_len = static["paths"], static["path_len"]
    lens = []
    for p, row in enumerate(paths):
        n = 0
        while n < path_len[p] and accepted_b[row[n + 1]]:
            n += 1
        lens.append(n)
    best = int(np.argmax(lens))             # first (lowest) index among the maxima
    return best, lens[best], paths[best][lens[best]]


def softmax(z_row):
    e = np.exp(z_row - z_row.max())
    return e / e.sum()


def mass_above(p, row, x):
    """Probability mass, under p (the row's softmax), of the tokens whose logit is strictly
    larger than token x's (row holds the logits)."""
    return float(p[row > row[x]].sum())


def typical_accept(logits, dtype, tokens, static, temperature, eps=0.09, delta=0.3):
    """logits [B,T,V] (stored dtype), tokens [B][T].  Returns a dict with best_candidate,
    accept_length, next_token (all [B]) plus per-child diagnostics:
      accepted [B,T] bool (root True), margin [B,T] = ln p(tok) - ln thr (nan at T=0 / root)."""
    return evaluate_posterior(logits, dtype, tokens, static, temperature, eps, delta)


def evaluate_posterior(logits, dtype, tokens, static, temperature, eps=0.09, delta=0.3,
                       top_p=1.0, sampling="typical", fast=False):
    """The candidate-filtering call of the cnnetsun page, evaluate_posterior(logits, candidates,
    temperature, posterior_threshold, posterior_alpha, top_p, sampling, fast), under these
    readings (the page names the last three arguments and defines none of them):
      sampling = "typical"  the typical-acceptance test above (top_p unused);
      sampling = "nucleus"  at temperature > 0, child c of node n is accepted iff it lies in the
                            top_p nucleus of p = softmax(l_n / T): the mass of the tokens whose
                            logit is strictly larger than tok(c)'s is below top_p
                            (margin = ln top_p - ln mass, +inf when the mass is 0);
      temperature 0         greedy in both modes;
      fast                  a faster evaluation of the same rule: no effect on the result.
    Returns the dict of typical_accept."""
    assert sampling in ("typical", "nucleus")
    assert 0.0 < top_p <= 1.0
    del fast
    B, T, V = logits.shape
    parent, children = static["parent"], static["children"]
    paths, path_len = static["paths"], static["path_len"]
    accepted = np.zeros((B, T), bool)
    margin = np.full((B, T), np.nan)
    argmax = np.full((B, T), -1, np.int64)
    H_all = np.full((B, T), np.nan)
    thr_all = np.full((B, T), np.nan)
    for b in range(B):
        accepted[b, 0] = True
        for n in range(T):
            if not children[n]:
                continue            # leaf rows are never needed for decisions
            row = _row_f64(logits, dtype, b, n)
            argmax[b, n] = _argmax_lowest(row)
            if temperature == 0:
                for c in children[n]:
                    accepted[b, c] = tokens[b][c] == argmax[b, n]
            elif sampling == "nucleus":
                p = softmax(row / temperature)
                for c in children[n]:
                    a = mass_above(p, row, tokens[b][c])
                    accepted[b, c] = a < top_p
                    margin[b, c] = np.log(top_p) - (np.log(a) if a > 0 else -np.inf)
            else:
                p, H, thr = row_threshold(row / temperature, eps, delta)
                H_all[b, n], thr_all[b, n] = H, thr
                for c in children[n]:
                    pc = p[tokens[b][c]]
                    accepted[b, c] = pc > thr
                    margin[b, c] = (np.log(pc) if pc > 0 else -np.inf) - np.log(thr)
    best = np.zeros(B, np.int32)
    alen = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        best[b], alen[b], last = scan_paths(static, accepted[b])
        nxt[b] = _argmax_lowest(_row_f64(logits, dtype, b, last))
    return dict(best_candidate=best, accept_length=alen, next_token=nxt, accepted=accepted,
                margin=margin, argmax=argmax, entropy=H_all, threshold=thr_all)
