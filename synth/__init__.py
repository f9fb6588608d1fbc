"""Seeded synthetic inputs for one Medusa verification step.

This module only draws numbers and lays them out.  It holds none of the
method's arithmetic (no heads, no top-k, no tree expansion, no attention, no
acceptance), so both the HIP path and the CPU oracle can be fed from it.

The workloads follow the shapes of the pages' examples: the three-head toy
model of the Ultralytics glossary page ("Medusa Heads", section on how the
heads predict), Vicuna-7B / Llama-3.1-8B / Vicuna-33B / 70B shapes from the
jisaku glossary page (benchmark table), 64-node sparse trees (Ultralytics
page, tree-attention section) and the 10 x 10 x 10 candidate count (jisaku
page, how-it-works section).  Real prompts, MT-Bench items and trained head
weights are not available; seeded Gaussians of the same shapes stand in.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gen_attention_inputs,
    gen_head_inputs,
    gen_root_tokens,
    gen_verif_logits,
    rng_for,
)
from .trees import load_tree_choices, sparse_tree_choices  # noqa: F401
