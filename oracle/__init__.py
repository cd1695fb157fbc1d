"""CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Importable only from the tests, the package's smoke check and the benchmark's
CPU-baseline leg. Nothing on the GPU path imports it; the two share no code.
"""
from .attention import (alibi_slopes, attention_bwd, attention_flops, attention_fwd, fp32_scale,
                        kv_head, merge_partials, visible, visible_pairs)

__all__ = ["attention_fwd", "attention_bwd", "attention_flops", "alibi_slopes", "fp32_scale", "kv_head",
           "merge_partials", "visible", "visible_pairs"]
