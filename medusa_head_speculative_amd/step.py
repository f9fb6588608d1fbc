"""One verification step on one stream: heads -> tree -> tree attention -> typical acceptance,
then (commit) the accepted candidate into the cache for the next step.

Holds the device buffers and workspaces of a fixed shape so the timed loop allocates nothing.
Inputs the step does not produce (the last hidden state, the tree tokens' Q/K/V inside the cache,
the verification logits, the root tokens) are given by the caller.
"""

import torch

from . import _lib


class VerifyStep:
    def __init__(self, *, B, hidden, vocab, K, topk, choices, Hq, Hkv, D, max_prefix_len,
                 device="cuda"):
        self.B, self.hidden, self.vocab, self.K, self.topk = B, hidden, vocab, K, topk
        self.Hq, self.Hkv, self.D, self.max_prefix_len = Hq, Hkv, D, max_prefix_len
        self.tree = _lib.Tree(choices, K, topk, device=device)
        T = self.tree.T
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_ids = torch.zeros((B, K, topk), **i32)
        self.topk_logits = torch.zeros((B, K, topk), dtype=torch.float32, device=device)
        self.logits = torch.zeros((B, K, vocab), dtype=torch.float32, device=device)
        self.tokens = torch.zeros((B, T), **i32)
        self.position_ids = torch.zeros((B, T), **i32)
        self.best = torch.zeros(B, **i32)
        self.accept_length = torch.zeros(B, **i32)
        self.next_token = torch.zeros(B, **i32)
        self.out_tokens = torch.zeros((B, self.tree.dims["dmax"] + 1), **i32)
        self.out_count = torch.zeros(B, **i32)
        self.new_prefix_len = torch.zeros(B, **i32)
        self.new_root = torch.zeros(B, **i32)
        self.ws_heads = _lib.workspace(_lib.medusa_heads_workspace(B, hidden, vocab, K, topk), device)
        self.ws_attn = _lib.workspace(_lib.tree_attention_workspace(B, Hq, Hkv, T, D, max_prefix_len), device)
        self.ws_acc = _lib.workspace(
            _lib.typical_accept_workspace(B, T, vocab, self.tree.dims["n_internal"]), device)

    def heads(self, h, w1, b1, w2, stream=None):
        """w1/w2 either [K, out, in] tensors or the flat packed tensors of pack_weights."""
        if w1.dim() == 1:
            _lib.medusa_heads_packed(h, w1, b1, w2, self.vocab, self.K, self.topk, self.topk_ids,
                                     self.ws_heads, logits=self.logits,
                                     topk_logits=self.topk_logits, stream=stream)
        else:
            _lib.medusa_heads(h, w1, b1, w2, self.topk, self.topk_ids, self.ws_heads,
                              logits=self.logits, topk_logits=self.topk_logits, stream=stream)

    def build(self, root_tokens, prefix_len, stream=None):
        _lib.build_tree(self.tree, self.topk_ids, root_tokens, prefix_len, self.tokens,
                        self.position_ids, stream=stream)

    def attention(self, q, k_cache, v_cache, prefix_len, out, stream=None):
        _lib.tree_attention(q, k_cache, v_cache, prefix_len, self.max_prefix_len, self.tree.mask,
                            out, self.ws_attn, stream=stream)

    def accept(self, verif_logits, temperature, eps=0.09, delta=0.3, next_token=True, stream=None):
        _lib.typical_accept(verif_logits, self.tokens, self.tree, temperature, eps, delta, self.best,
                            self.accept_length, self.ws_acc,
                            next_token=self.next_token if next_token else None, stream=stream)

    def heads_and_tree(self, h, w1, b1, w2, root_tokens, prefix_len, stream=None):
        """heads then the tree tokens and position ids; once the tree is on the device, in the
        same launches (medusa_heads_build_tree)."""
        if not self.tree.static_ready:
            self.heads(h, w1, b1, w2, stream)
            self.build(root_tokens, prefix_len, stream)
            return
        _lib.medusa_heads_build_tree(h, w1, b1, w2, self.vocab, self.K, self.topk, self.tree,
                                     root_tokens, prefix_len, self.topk_ids, self.tokens,
                                     self.position_ids, self.ws_heads, logits=self.logits,
                                     topk_logits=self.topk_logits, stream=stream)

    def run(self, *, h, w1, b1, w2, root_tokens, prefix_len, q, k_cache, v_cache, attn_out,
            verif_logits, temperature, eps=0.09, delta=0.3, stream=None):
        self.heads_and_tree(h, w1, b1, w2, root_tokens, prefix_len, stream)
        self.attention(q, k_cache, v_cache, prefix_len, attn_out, stream)
        self.accept(verif_logits, temperature, eps, delta, stream=stream)

    def capture(self, **run_kwargs):
        """run(**run_kwargs) recorded into a HIP graph (a torch.cuda.CUDAGraph), to be replayed
        with the same buffers: one host call per step instead of one per launch, for steps small
        enough that issuing the launches costs more than running them.  The step allocates,
        copies and clears nothing once the tree is on the device (an eager run first puts it
        there), so the graph holds kernel nodes only.  Replays read whatever the input buffers
        hold at replay time."""
        if not self.tree.static_ready:
            self.run(**run_kwargs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            self.run(**run_kwargs)
        torch.cuda.current_stream().wait_stream(side)
        return graph

    def commit(self, k_cache, v_cache, prefix_len, hidden=None, next_hidden=None, stream=None):
        """After accept: emit the accepted tokens (out_tokens, out_count), move their K/V rows
        into place, and set new_prefix_len / new_root (and next_hidden from hidden)."""
        _lib.commit_accepted(self.tree, self.best, self.accept_length, self.tokens,
                             self.next_token, k_cache, v_cache, prefix_len, self.new_prefix_len,
                             self.out_tokens, self.out_count, new_root=self.new_root,
                             hidden=hidden, next_hidden=next_hidden, stream=stream)
