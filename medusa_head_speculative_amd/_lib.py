"""ctypes binding of libmedusa_hip.so.  Argument marshalling only: every step runs in the library
(HIP kernels; the static tree and the sparse-tree choice are its host code).

Tensors are torch tensors on the current HIP device (bf16 tensors may be torch.bfloat16 or
int16/uint16 bit patterns); the functions pass their data pointers and the current stream to the
C ABI declared in include/medusa.h and raise MedusaError on a non-zero status.
"""

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(HERE, "libmedusa_hip.so")

F32, BF16 = 0, 1
STATUS = {0: "OK", -1: "ERR_ARG", -2: "ERR_SHAPE", -3: "ERR_DTYPE", -4: "ERR_TREE",
          -5: "ERR_WORKSPACE", -6: "ERR_HIP", -7: "ERR_UNSUPPORTED"}


class MedusaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class medusa_tree(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("W", ctypes.c_int), ("n_paths", ctypes.c_int),
                ("dmax", ctypes.c_int), ("n_internal", ctypes.c_int), ("max_rank", ctypes.c_int),
                ("mask", ctypes.c_void_p), ("parent", ctypes.c_void_p),
                ("depth", ctypes.c_void_p), ("rank", ctypes.c_void_p),
                ("paths", ctypes.c_void_p), ("path_len", ctypes.c_void_p),
                ("child_ptr", ctypes.c_void_p), ("child_idx", ctypes.c_void_p),
                ("internal", ctypes.c_void_p)]


EXPORTS = ["medusa_last_error", "medusa_heads_workspace", "medusa_heads", "medusa_tree_dims",
           "build_tree", "tree_attention_workspace", "tree_attention",
           "typical_accept_workspace", "typical_accept", "medusa_set_kernel_events",
           "medusa_heads_packed", "medusa_packed_weight_bytes", "medusa_pack_weights",
           "medusa_stream_read", "commit_accepted", "tree_attention_rope_workspace",
           "tree_attention_rope", "medusa_sparse_tree", "medusa_heads_ex_workspace",
           "medusa_heads_ex", "typical_accept_noalloc", "evaluate_posterior_workspace",
           "evaluate_posterior", "medusa_heads_build_tree"]

SAMPLING = {"typical": 0, "nucleus": 1}

KERNELS = ["heads_w1", "heads_w2", "topk", "tree_gather", "attention", "attn_combine", "accept",
           "commit", "rope"]

_lib = None


def load():
    """Load libmedusa_hip.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is missing: build it with "
                          "`python -m medusa_head_speculative_amd.build`")
    L = ctypes.CDLL(LIBPATH)
    vp, i, l, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_float, ctypes.c_size_t
    tp = ctypes.POINTER(medusa_tree)
    L.medusa_last_error.restype = ctypes.c_char_p
    L.medusa_last_error.argtypes = []
    L.medusa_heads_workspace.restype = sz
    L.medusa_heads_workspace.argtypes = [i, i, l, i, i]
    L.medusa_heads.restype = i
    L.medusa_heads.argtypes = [vp, vp, vp, vp, i, i, i, l, i, i, vp, vp, vp, vp, sz, vp]
    L.medusa_tree_dims.restype = i
    L.medusa_tree_dims.argtypes = [vp, i, i, i, i, tp]
    L.build_tree.restype = i
    L.build_tree.argtypes = [vp, i, i, i, i, vp, vp, vp, i, i, tp, vp, vp, vp]
    L.tree_attention_workspace.restype = sz
    L.tree_attention_workspace.argtypes = [i, i, i, i, i, i]
    L.tree_attention.restype = i
    L.tree_attention.argtypes = [vp, vp, vp, i, vp, i, l, vp, i, i, i, i, i, f, vp, vp, sz, vp]
    L.typical_accept_workspace.restype = sz
    L.typical_accept_workspace.argtypes = [i, i, l, i]
    L.typical_accept.restype = i
    L.typical_accept.argtypes = [vp, i, i, i, l, vp, tp, f, f, f, vp, vp, vp, vp, sz, vp]
    L.medusa_heads_build_tree.restype = i
    L.medusa_heads_build_tree.argtypes = [vp, vp, vp, vp, i, i, i, i, l, i, i, tp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, sz, vp]
    L.evaluate_posterior_workspace.restype = sz
    L.evaluate_posterior_workspace.argtypes = [i, l, tp, i]
    L.evaluate_posterior.restype = i
    L.evaluate_posterior.argtypes = [vp, i, i, i, l, vp, tp, f, f, f, f, i, i, vp, vp, vp, vp, sz,
                                     vp]
    L.typical_accept_noalloc.restype = i
    L.typical_accept_noalloc.argtypes = [vp, i, i, i, l, vp, tp, f, f, f, vp, vp, vp, vp]
    L.medusa_set_kernel_events.restype = i
    L.medusa_heads_packed.restype = i
    L.medusa_heads_packed.argtypes = [vp, vp, vp, vp, i, i, l, i, i, vp, vp, vp, vp, sz, vp]
    L.medusa_packed_weight_bytes.restype = sz
    L.medusa_packed_weight_bytes.argtypes = [i, l, i]
    L.medusa_pack_weights.restype = i
    L.medusa_pack_weights.argtypes = [vp, i, l, i, vp, vp]
    L.medusa_set_kernel_events.argtypes = [i, vp, vp]
    L.medusa_stream_read.restype = i
    L.medusa_stream_read.argtypes = [vp, sz, vp, vp]
    L.tree_attention_rope_workspace.restype = sz
    L.tree_attention_rope_workspace.argtypes = [i, i, i, i, i, i]
    L.tree_attention_rope.restype = i
    L.tree_attention_rope.argtypes = [vp, vp, vp, i, vp, i, l, vp, vp, f, i, i, i, i, i, f, vp,
                                      vp, sz, vp]
    L.medusa_heads_ex_workspace.restype = sz
    L.medusa_heads_ex_workspace.argtypes = [i, i, l, i, i, i, i]
    L.medusa_heads_ex.restype = i
    L.medusa_heads_ex.argtypes = [vp, vp, vp, vp, vp, f, vp, i, i, i, i, l, i, i, i, vp, vp, vp,
                                  vp, sz, vp]
    L.medusa_sparse_tree.restype = i
    L.medusa_sparse_tree.argtypes = [vp, i, i, i, vp, vp]
    L.commit_accepted.restype = i
    L.commit_accepted.argtypes = [ctypes.POINTER(medusa_tree), i, vp, vp, vp, vp, vp, vp, i, i, l,
                                  i, vp, vp, vp, vp, vp, vp, i, vp, vp]
    _lib = L
    return L


def _check(rc):
    if rc != 0:
        raise MedusaError(rc, load().medusa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace(nbytes, device=None):
    """A workspace of at least `nbytes` bytes (zero-filled; the kernels need no particular contents)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------------------------------------
def medusa_heads_workspace(B, hidden, vocab, K, topk):
    return load().medusa_heads_workspace(B, hidden, vocab, K, topk)


def medusa_heads(h, w1, b1, w2, topk, topk_ids, ws, logits=None, topk_logits=None, stream=None):
    """h [B,Hd]; w1 [K,Hd,Hd]; b1 [K,Hd]; w2 [K,V,Hd]; topk_ids [B,K,topk] int32 (out)."""
    B, hd = h.shape
    K, V = w2.shape[0], w2.shape[1]
    _check(load().medusa_heads(_ptr(h), _ptr(w1), _ptr(b1), _ptr(w2), dtype_code(h), B, hd, V, K,
                               topk, _ptr(logits), _ptr(topk_ids), _ptr(topk_logits), _ptr(ws),
                               ws.numel(), _stream(stream)))


def pack_weights(w, stream=None):
    """w [K, rows, hidden] bf16 -> packed bf16 tensor (flat) for medusa_heads_packed."""
    K, rows, hd = w.shape
    n = load().medusa_packed_weight_bytes(K, rows, hd)
    if n == 0:
        raise MedusaError(-2, f"cannot pack a [{K}, {rows}, {hd}] weight")
    out = torch.empty(n // 2, dtype=torch.bfloat16, device=w.device)
    _check(load().medusa_pack_weights(_ptr(w), K, rows, hd, _ptr(out), _stream(stream)))
    return out


def medusa_heads_packed(h, w1_packed, b1, w2_packed, vocab, K, topk, topk_ids, ws, logits=None,
                        topk_logits=None, stream=None):
    """As medusa_heads with weights from pack_weights (bf16)."""
    B, hd = h.shape
    _check(load().medusa_heads_packed(_ptr(h), _ptr(w1_packed), _ptr(b1), _ptr(w2_packed), B, hd,
                                      vocab, K, topk, _ptr(logits), _ptr(topk_ids),
                                      _ptr(topk_logits), _ptr(ws), ws.numel(), _stream(stream)))


# ---------------------------------------------------------------------------------------------
def medusa_heads_ex_workspace(B, hidden, vocab, K, n_blocks, layernorm, topk):
    return load().medusa_heads_ex_workspace(B, hidden, vocab, K, n_blocks, 1 if layernorm else 0,
                                            topk)


def medusa_heads_ex(h, w1, b1, w2, vocab, K, n_blocks, topk, topk_ids, ws, ln_gamma=None,
                    ln_beta=None, ln_eps=1e-5, packed=False, logits=None, topk_logits=None,
                    stream=None):
    """Heads of n_blocks residual blocks (optionally with LayerNorm).  w1 [K, n_blocks, Hd, Hd]
    (or pack_weights of its [K * n_blocks, Hd, Hd] view with packed=True), b1 [K, n_blocks, Hd],
    ln_gamma / ln_beta [K, n_blocks, Hd] or None, w2 [K, V, Hd] (or packed)."""
    B, hd = h.shape
    _check(load().medusa_heads_ex(_ptr(h), _ptr(w1), _ptr(b1), _ptr(ln_gamma), _ptr(ln_beta),
                                  ln_eps, _ptr(w2), dtype_code(h), 1 if packed else 0, B, hd,
                                  vocab, K, n_blocks, topk, _ptr(logits), _ptr(topk_ids),
                                  _ptr(topk_logits), _ptr(ws), ws.numel(), _stream(stream)))


def _choices_array(choices, max_depth=None):
    import numpy as np
    md = max_depth or max(len(c) for c in choices)
    a = np.full((len(choices), md), -1, np.int32)
    for r, c in enumerate(choices):
        a[r, :len(c)] = c
    return a, md


class Tree:
    """Device arrays of one fixed tree (medusa_tree) plus its dims.  Built once per tree."""

    def __init__(self, choices, K, topk, device="cuda"):
        L = load()
        self.choices, self.max_depth = _choices_array(choices)
        self.K, self.topk = K, topk
        self.c = medusa_tree()
        _check(L.medusa_tree_dims(ctypes.c_void_p(self.choices.ctypes.data), len(choices),
                                  self.max_depth, K, topk, ctypes.byref(self.c)))
        T, W, P, dm, ni = self.c.T, self.c.W, self.c.n_paths, self.c.dmax, self.c.n_internal
        i32 = dict(dtype=torch.int32, device=device)
        self.mask = torch.zeros((T, W), dtype=torch.int64, device=device)
        self.parent = torch.zeros(T, **i32)
        self.depth = torch.zeros(T, **i32)
        self.rank = torch.zeros(T, **i32)
        self.paths = torch.zeros((P, dm + 1), **i32)
        self.path_len = torch.zeros(P, **i32)
        self.child_ptr = torch.zeros(T + 1, **i32)
        self.child_idx = torch.zeros(max(T - 1, 1), **i32)
        self.internal = torch.zeros(ni, **i32)
        for name in ("mask", "parent", "depth", "rank", "paths", "path_len", "child_ptr",
                     "child_idx", "internal"):
            setattr(self.c, name, getattr(self, name).data_ptr())
        self.static_ready = 0

    @property
    def T(self):
        return self.c.T

    @property
    def dims(self):
        c = self.c
        return dict(T=c.T, W=c.W, n_paths=c.n_paths, dmax=c.dmax, n_internal=c.n_internal,
                    max_rank=c.max_rank)


def medusa_heads_build_tree(h, w1, b1, w2, vocab, K, topk, tree, root_tokens, prefix_len,
                            topk_ids, tokens, position_ids, ws, logits=None, topk_logits=None,
                            stream=None):
    """medusa_heads (w1/w2 [K, out, in]) or medusa_heads_packed (flat packed w1/w2) and the
    tree gather of build_tree in the same launches; the tree must already be uploaded."""
    if not tree.static_ready:
        raise ValueError("upload the tree first (one build_tree call)")
    B, hd = h.shape
    packed = 1 if w1.dim() == 1 else 0
    _check(load().medusa_heads_build_tree(_ptr(h), _ptr(w1), _ptr(b1), _ptr(w2), dtype_code(h),
                                          packed, B, hd, vocab, K, topk, ctypes.byref(tree.c),
                                          _ptr(root_tokens), _ptr(prefix_len), _ptr(logits),
                                          _ptr(topk_ids), _ptr(topk_logits), _ptr(tokens),
                                          _ptr(position_ids), _ptr(ws), ws.numel(),
                                          _stream(stream)))


def build_tree(tree, topk_ids, root_tokens, prefix_len, tokens, position_ids, stream=None):
    """First call uploads the static arrays (host waits); later calls only gather."""
    B = root_tokens.shape[0]
    _check(load().build_tree(ctypes.c_void_p(tree.choices.ctypes.data), tree.choices.shape[0],
                             tree.max_depth, tree.K, tree.topk, _ptr(topk_ids), _ptr(root_tokens),
                             _ptr(prefix_len), B, tree.static_ready, ctypes.byref(tree.c),
                             _ptr(tokens), _ptr(position_ids), _stream(stream)))
    tree.static_ready = 1


# ---------------------------------------------------------------------------------------------
def tree_attention_workspace(B, Hq, Hkv, T, D, max_prefix_len):
    return load().tree_attention_workspace(B, Hq, Hkv, T, D, max_prefix_len)


def tree_attention(q, k_cache, v_cache, prefix_len, max_prefix_len, mask, out, ws, scale=0.0,
                   stream=None):
    """q/out [B,Hq,T,D]; caches [B,Hkv,Lcap,D]; mask [T,W] int64 bit words."""
    B, Hq, T, D = q.shape
    Hkv, lcap = k_cache.shape[1], k_cache.shape[2]
    _check(load().tree_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), dtype_code(q),
                                 _ptr(prefix_len), max_prefix_len, lcap, _ptr(mask), B, Hq, Hkv, T,
                                 D, scale, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def tree_attention_rope_workspace(B, Hq, Hkv, T, D, max_prefix_len):
    return load().tree_attention_rope_workspace(B, Hq, Hkv, T, D, max_prefix_len)


def tree_attention_rope(q, k_cache, v_cache, prefix_len, max_prefix_len, mask, position_ids,
                        out, ws, rope_base=10000.0, scale=0.0, stream=None):
    """tree_attention after rotating the tree tokens' q (into ws) and their k_cache rows (in
    place) at position_ids [B,T]."""
    B, Hq, T, D = q.shape
    Hkv, lcap = k_cache.shape[1], k_cache.shape[2]
    _check(load().tree_attention_rope(_ptr(q), _ptr(k_cache), _ptr(v_cache), dtype_code(q),
                                      _ptr(prefix_len), max_prefix_len, lcap, _ptr(mask),
                                      _ptr(position_ids), rope_base, B, Hq, Hkv, T, D, scale,
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


# ---------------------------------------------------------------------------------------------
def typical_accept_workspace(B, T, V, n_internal):
    return load().typical_accept_workspace(B, T, V, n_internal)


def typical_accept(logits, tokens, tree, temperature, posterior_threshold, posterior_alpha,
                   best_candidate, accept_length, ws, next_token=None, stream=None):
    """logits [B,T,V]; tokens [B,T] int32; outputs int32 [B]."""
    B, T, V = logits.shape
    _check(load().typical_accept(_ptr(logits), dtype_code(logits), B, T, V, _ptr(tokens),
                                 ctypes.byref(tree.c), temperature, posterior_threshold,
                                 posterior_alpha, _ptr(best_candidate), _ptr(accept_length),
                                 _ptr(next_token), _ptr(ws), ws.numel(), _stream(stream)))


def evaluate_posterior_workspace(B, vocab, tree, sampling="typical"):
    return load().evaluate_posterior_workspace(B, vocab, ctypes.byref(tree.c), SAMPLING[sampling])


def evaluate_posterior(logits, tokens, tree, temperature, posterior_threshold, posterior_alpha,
                       best_candidate, accept_length, ws, top_p=1.0, sampling="typical",
                       fast=False, next_token=None, stream=None):
    """typical_accept with the page's top_p / sampling / fast arguments ("typical" or
    "nucleus"; see include/medusa.h for their readings)."""
    B, T, V = logits.shape
    _check(load().evaluate_posterior(_ptr(logits), dtype_code(logits), B, T, V, _ptr(tokens),
                                     ctypes.byref(tree.c), temperature, posterior_threshold,
                                     posterior_alpha, top_p, SAMPLING[sampling], 1 if fast else 0,
                                     _ptr(best_candidate), _ptr(accept_length), _ptr(next_token),
                                     _ptr(ws), ws.numel(), _stream(stream)))


def typical_accept_noalloc(logits, tokens, tree, temperature, posterior_threshold,
                           posterior_alpha, best_candidate, accept_length, next_token=None,
                           stream=None):
    """typical_accept without a workspace: the library's per-GPU scratch array holds the
    intermediates (for callers that cannot allocate; overlapping calls on one GPU race)."""
    B, T, V = logits.shape
    _check(load().typical_accept_noalloc(_ptr(logits), dtype_code(logits), B, T, V, _ptr(tokens),
                                         ctypes.byref(tree.c), temperature, posterior_threshold,
                                         posterior_alpha, _ptr(best_candidate),
                                         _ptr(accept_length), _ptr(next_token), _stream(stream)))


def commit_accepted(tree, best_candidate, accept_length, tokens, next_token, k_cache, v_cache,
                    prefix_len, new_prefix_len, out_tokens, out_count, new_root=None, hidden=None,
                    next_hidden=None, stream=None):
    """Emit the accepted tokens, compact their K/V rows in the cache (in place), advance the
    prefix and hand over the next root and hidden state (see include/medusa.h).  Caches
    [B, Hkv, lcap, D]; out_tokens [B, dmax + 1]; hidden [B, T, Hd] / next_hidden [B, Hd]."""
    B, Hkv, lcap, D = k_cache.shape
    hd = 0 if hidden is None else hidden.shape[2]
    _check(load().commit_accepted(ctypes.byref(tree.c), B, _ptr(best_candidate),
                                  _ptr(accept_length), _ptr(tokens), _ptr(next_token),
                                  _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), Hkv, lcap, D,
                                  _ptr(prefix_len), _ptr(new_prefix_len), _ptr(out_tokens),
                                  _ptr(out_count), _ptr(new_root), _ptr(hidden), hd,
                                  _ptr(next_hidden), _stream(stream)))


def sparse_tree(accuracy, N):
    """The N-node choice list of largest expected accept length for per-head rank accuracies
    accuracy [K][topk] (host).  Returns (choices as lists of ranks in node order, expectation)."""
    acc = np.ascontiguousarray(accuracy, dtype=np.float64)
    K, topk = acc.shape
    out = np.empty((N, K), np.int32)
    e = ctypes.c_double()
    _check(load().medusa_sparse_tree(acc.ctypes.data, K, topk, N, out.ctypes.data,
                                     ctypes.byref(e)))
    return [[int(r) for r in row if r >= 0] for row in out], e.value


# ---------------------------------------------------------------------------------------------
def set_kernel_events(kernel, before=None, after=None):
    """Measurement hook: record torch.cuda.Events around every launch of `kernel` (a name from
    KERNELS) on this thread; None clears it.  The events must have been recorded once (so that
    torch has created them)."""
    which = KERNELS.index(kernel)
    b = ctypes.c_void_p(before.cuda_event) if before is not None else None
    a = ctypes.c_void_p(after.cuda_event) if after is not None else None
    _check(load().medusa_set_kernel_events(which, b, a))


def stream_read(buf, sink, stream=None):
    """Measurement: one streaming read of the whole of `buf` (a contiguous device tensor whose
    size in bytes is a multiple of 16) by the library's plain read kernel; `sink` is a device
    int32 tensor of at least one element that the kernel may write."""
    nbytes = buf.numel() * buf.element_size()
    _check(load().medusa_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
