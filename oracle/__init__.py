"""fp64 CPU oracle for one Medusa verification step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU
baseline, never by the HIP library or its Python binding.  It shares no code with them.

Parts: heads + top-k (heads.py, C loops in medusa_oracle.c; several residual blocks with
optional LayerNorm in head_blocks.py), the candidate tree (tree.py),
tree-masked attention (attention.py, C loops) and its rotary position embedding at depth
positions (rope.py), typical acceptance (accept.py) and the commit of the accepted candidate into
the cache (commit.py).
"""

from . import _clib  # noqa: F401
from .accept import evaluate_posterior, row_threshold, typical_accept  # noqa: F401
from .attention import tree_attention  # noqa: F401
from .commit import commit  # noqa: F401
from .head_blocks import heads_blocks  # noqa: F401
from .heads import heads, project, topk, topk_ties  # noqa: F401
from .rope import rope, rotate_tree, tree_attention_rope  # noqa: F401
from .tree import TreeError, build_static, canonical, gather  # noqa: F401


def build():
    _clib.build(force=True)
