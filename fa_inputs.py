"""Seeded synthetic inputs for the attention forward pass.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic, so both the GPU path's tests/bench and
the CPU oracle's tests may use it.

Distribution: every page that builds attention inputs draws Q, K and V iid from
N(0, 1) (the Lab 3 page "Tiled attention with online softmax", the NumPy
tiled-block guide's "Synthetic Data" step, the PyTorch SDPA usage example on the
"Flash Attention" overview page). The generator is NumPy's PCG64
(`numpy.random.default_rng`), the one the Lab 3 page and the NumPy tiled-block
guide use.

Recipe for a config (B, H, S, D, dtype, seed):
  rng = default_rng(seed); Q, K, V drawn in that order, each as
  rng.standard_normal((B, H, S, D), dtype=float32), then rounded to the storage
  dtype with round-to-nearest-even (torch's `.to`). With grouped key/value
  heads, K and V are drawn with H_kv heads instead of H.
The single-head fp32 worked-example config instead reproduces the Lab 3 page's
own draw: rng.normal(size=(64, 16)) three times in float64, then cast to fp32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str          # "f32" | "f16" | "bf16"
    causal: bool
    scale: float
    window: int = 0
    n_sink: int = 0
    seed: int = 0
    lab3_draw: bool = False   # reproduce the Lab 3 page's (64, 16) float64 draw
    H_kv: int = 0             # key/value heads (0: same as H)
    alibi: bool = False       # ALiBi bias with the Lesson 91 deck's slopes
    n_split: int = 1          # key ranges per query block (partials + merge)
    backward: bool = False    # time the backward pass (gradients from a forward's O, LSE)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H


# The five workloads the attention forward pass is measured and checked on.
WORKLOADS = {
    # Lab 3 worked example: single head, causal, n=64, d=16, seed 0.
    "causal_b1h1s64d16_f32": Workload("causal_b1h1s64d16_f32", 1, 1, 64, 16, "f32", True,
                                      1.0 / math.sqrt(16), lab3_draw=True),
    # The SDPA usage example's shape [2, 8, 1024, 64] in fp16, no mask.
    "noncausal_b2h8s1024d64_f16": Workload("noncausal_b2h8s1024d64_f16", 2, 8, 1024, 64, "f16",
                                           False, 1.0 / 8.0),
    # Headline: causal MHA, bf16.
    "causal_b4h16s4096d128_bf16": Workload("causal_b4h16s4096d128_bf16", 4, 16, 4096, 128,
                                           "bf16", True, 1.0 / math.sqrt(128)),
    # One GPU's share of a long-sequence layer.
    "causal_b1h32s16384d128_bf16": Workload("causal_b1h32s16384d128_bf16", 1, 32, 16384, 128,
                                            "bf16", True, 1.0 / math.sqrt(128)),
    # Causal + sliding window 1024 + 4 always-attended sink keys.
    "window1024_sink4_b8h32s8192d128_bf16": Workload(
        "window1024_sink4_b8h32s8192d128_bf16", 8, 32, 8192, 128, "bf16", True,
        1.0 / math.sqrt(128), window=1024, n_sink=4),
}
HEADLINE = "causal_b4h16s4096d128_bf16"

# Variants of the headline shape for the grouped-head and ALiBi extensions
# (Lesson 91 deck: GQA with groups of 8 query heads, ALiBi slopes per head).
EXTENSIONS = {
    "gqa_causal_b4h16kv2s4096d128_bf16": Workload(
        "gqa_causal_b4h16kv2s4096d128_bf16", 4, 16, 4096, 128, "bf16", True,
        1.0 / math.sqrt(128), H_kv=2),
    "alibi_causal_b4h16s4096d128_bf16": Workload(
        "alibi_causal_b4h16s4096d128_bf16", 4, 16, 4096, 128, "bf16", True,
        1.0 / math.sqrt(128), alibi=True),
    # Few heads: 8 heads x 16 query blocks fill a sixth of the CUs; splitting
    # the keys of each query block four ways fills them.
    "split4_causal_b1h8s4096d128_bf16": Workload(
        "split4_causal_b1h8s4096d128_bf16", 1, 8, 4096, 128, "bf16", True,
        1.0 / math.sqrt(128), n_split=4),
    # The backward pass of the headline shape (dO drawn after Q, K, V).
    "bwd_causal_b4h16s4096d128_bf16": Workload(
        "bwd_causal_b4h16s4096d128_bf16", 4, 16, 4096, 128, "bf16", True,
        1.0 / math.sqrt(128), backward=True),
}
ALL_WORKLOADS = {**WORKLOADS, **EXTENSIONS}


def make_qkv(B: int, H: int, S: int, D: int, dtype: str, seed: int = 0,
             lab3_draw: bool = False, H_kv: int = 0):
    """Return (q, k, v) as contiguous CPU torch tensors in `dtype`: q [B, H, S, D],
    k and v [B, H_kv, S, D] (H_kv = 0 means H)."""
    rng = np.random.default_rng(seed)
    Hk = H_kv or H
    if lab3_draw:
        if (B, H, Hk) != (1, 1, 1):
            raise ValueError("the Lab 3 draw is a single (S, D) head")
        arrs = [rng.normal(size=(S, D)) for _ in range(3)]           # float64
        arrs = [a.reshape(1, 1, S, D) for a in arrs]
    else:
        arrs = [rng.standard_normal(size=(B, h, S, D), dtype=np.float32) for h in (H, Hk, Hk)]
    out = []
    for a in arrs:
        t = torch.from_numpy(np.ascontiguousarray(a)).to(DTYPES[dtype]).contiguous()
        out.append(t)
    return tuple(out)


def make_qkv_device(S: int, D: int, dtype: str, seed: int, device) -> tuple:
    """(q, k, v) of one head, [1, 1, S, D] in `dtype`, drawn N(0, 1) by torch's
    generator on `device` (for sequences too long to draw on the host); rows
    are drawn in chunks so the fp32 staging stays small."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(3):
        t = torch.empty((1, 1, S, D), dtype=DTYPES[dtype], device=device)
        for r0 in range(0, S, 1 << 20):
            r1 = min(S, r0 + (1 << 20))
            t[0, 0, r0:r1] = torch.randn((r1 - r0, D), generator=g, device=device).to(DTYPES[dtype])
        out.append(t)
    return tuple(out)


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.S, w.D, w.dtype, w.seed, w.lab3_draw, w.H_kv)


def make_dout(w: Workload):
    """The upstream gradient dO [B, H, S, D] of a backward workload: N(0, 1) from
    default_rng(seed + 1), rounded to the dtype like Q, K, V."""
    rng = np.random.default_rng(w.seed + 1)
    a = rng.standard_normal(size=(w.B, w.H, w.S, w.D), dtype=np.float32)
    return torch.from_numpy(a).to(DTYPES[w.dtype]).contiguous()


def lab3_example():
    """The Lab 3 page's exact inputs: default_rng(0), three (64, 16) float64 N(0,1) draws."""
    rng = np.random.default_rng(0)
    return tuple(rng.normal(size=(64, 16)) for _ in range(3))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a stored tensor (any of the three dtypes) to a float64 array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
