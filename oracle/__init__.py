"""CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Importable only from the tests, the package's smoke check and the benchmark's
CPU-baseline leg. Nothing on the GPU path imports it; the two share no code.
"""
from .attention import (attention_flops, attention_fwd, fp32_scale,
                        visible, visible_pairs)

__all__ = ["attention_fwd", "attention_flops", "fp32_scale", "visible",
           "visible_pairs"]
