"""MI355X-native Medusa verification step: Python binding of libmedusa_hip.so.

Entry points (same names as the C ABI in include/medusa.h): medusa_heads, build_tree,
tree_attention, typical_accept, commit_accepted, their *_workspace queries, the Tree helper (device arrays of a
fixed tree) and VerifyStep (the four calls chained on one stream).
"""

from ._lib import (  # noqa: F401
    BF16,
    EXPORTS,
    F32,
    KERNELS,
    MedusaError,
    Tree,
    build_tree,
    commit_accepted,
    evaluate_posterior,
    evaluate_posterior_workspace,
    load,
    medusa_heads,
    medusa_heads_build_tree,
    medusa_heads_ex,
    medusa_heads_ex_workspace,
    medusa_heads_packed,
    pack_weights,
    medusa_heads_workspace,
    set_kernel_events,
    sparse_tree,
    stream_read,
    tree_attention,
    tree_attention_rope,
    tree_attention_rope_workspace,
    tree_attention_workspace,
    typical_accept,
    typical_accept_noalloc,
    typical_accept_workspace,
    workspace,
)
from .step import VerifyStep  # noqa: F401
