"""The five synthetic workloads of one verification step.

Shapes come from the pages: the toy model (hidden 256, vocab 1000, 3 heads)
of the Ultralytics "Medusa Heads" page, the model/head-count table of the
jisaku glossary page (benchmark section), top-10 per head (jisaku page,
how-it-works: k = 10..50), 64-node sparse trees (Ultralytics page,
tree-attention section) and the full 10+100+1000 tree (K=3, k=10 gives up
to 1000 candidates, jisaku page, how-it-works).
"""

from dataclasses import dataclass, field
import math


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    dtype: str          # "f32" or "bf16": element type of every tensor input
    B: int              # batch (independent sequences)
    Hd: int             # hidden size
    V: int              # vocab size
    K: int              # Medusa heads
    topk: int           # candidates kept per head
    Hq: int             # query heads of the attention layer
    Hkv: int            # key/value heads
    D: int              # head dim
    L: int              # prefix length (tokens already in the KV cache)
    tree: str           # tree choice list name (synth/trees/<tree>.json)
    temps: tuple        # acceptance temperatures exercised
    boost_p: float      # probability a node's own token is boosted in its verifying row
    seed: int
    w_std: float        # std of W1, b1, W2
    eps: float = 0.09   # posterior_threshold (cnnetsun page, architecture section)
    delta: float = 0.3  # posterior_alpha
    boost: float = 6.0
    logit_std: float = 2.0
    extra: dict = field(default_factory=dict)

    @property
    def esize(self):
        return 4 if self.dtype == "f32" else 2


CONFIGS = [
    Config(0, "tiny_fp32", "f32", B=1, Hd=256, V=1000, K=3, topk=3, Hq=4, Hkv=4, D=64,
           L=128, tree="c0", temps=(0.7,), boost_p=0.7, seed=0, w_std=0.02),
    Config(1, "vicuna7b_bf16", "bf16", B=1, Hd=4096, V=32000, K=4, topk=10, Hq=32, Hkv=32,
           D=128, L=1024, tree="c1", temps=(0.0, 0.7), boost_p=0.7, seed=1,
           w_std=1.0 / math.sqrt(4096)),
    Config(2, "llama31_8b_bf16", "bf16", B=1, Hd=4096, V=128256, K=5, topk=10, Hq=32, Hkv=8,
           D=128, L=4096, tree="c2", temps=(0.0, 0.7), boost_p=0.6, seed=2,
           w_std=1.0 / math.sqrt(4096)),
    Config(3, "vicuna33b_b8_bf16", "bf16", B=8, Hd=6656, V=32000, K=3, topk=10, Hq=52, Hkv=52,
           D=128, L=2048, tree="c3", temps=(0.7,), boost_p=0.7, seed=3,
           w_std=1.0 / math.sqrt(6656)),
    Config(4, "llama70b_layer_b4_bf16", "bf16", B=4, Hd=8192, V=128256, K=3, topk=10, Hq=64,
           Hkv=8, D=128, L=8192, tree="c4", temps=(0.0, 0.7), boost_p=0.6, seed=4,
           w_std=1.0 / math.sqrt(8192)),
]


def get_config(i):
    return CONFIGS[i]


def custom(**kw):
    """A Config for tests (ragged shapes, fuzz); unspecified fields take c0's values."""
    base = dict(idx=-1, name="custom", dtype="f32", B=1, Hd=256, V=1000, K=3, topk=3, Hq=4,
                Hkv=4, D=64, L=128, tree="c0", temps=(0.7,), boost_p=0.7, seed=0, w_std=0.02)
    base.update(kw)
    return Config(**base)
