"""fp64 CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module. The GPU path never calls it, imports it or shares code
with it.

What it computes. The method on the pages reaches the ordinary attention result
exactly -- the "Flash Attention" overview page's "Mathematical Equivalence"
section states that it is not an approximation, and the Lab 3 page ("Tiled
attention with online softmax") sets out to show that tiling equals ordinary
attention -- so the oracle is the plain definition, written out:

    O   = softmax(Q K^T * scale + mask) V
    LSE = log-sum-exp of each masked, scaled score row (natural log)

Sources of the definition:
  * "Flash Attention" overview page, "The Problem with Standard Attention":
    Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V.
  * Lab 3 page, its `reference` function: scores scaled by 1/sqrt(d), the
    lower-triangular (diagonal-included) causal mask applied as -inf, softmax
    with the row max subtracted, then P @ V.
  * NumPy tiled-block guide, Step 2 ("Naive Scaled Dot-Product Attention"):
    the same without a mask.
  * The logsumexp output: the NumPy build guide (Step 5 comment) names the
    cross-tile logsumexp that full FlashAttention tracks.

Readings where the pages are silent (each also listed in the design notes):
  R1 scale: the value the C ABI receives is an fp32 number, so the oracle
     rounds `scale` to fp32 first and then works in fp64 with that value.
  R2 causal: key j is visible to query i iff j <= i (diagonal kept), as in the
     Lab 3 mask and its block loop.
  R3 sliding window of width W (W > 0): key j is visible iff i - j < W, i.e.
     the W most recent keys including i itself (the Lab 3 exercise on sinks and
     windows defers the definition to a chapter that is not on the pages).
  R4 sinks: the first n_sink key positions stay visible to every query that
     causality allows (j <= i), whatever the window; n_sink only matters with
     a window. Visible set = window keys UNION sink keys.
  R5 a window without the causal mask is not a defined operation (rejected).
  R6 LSE_i = m_i + ln(l_i) in the scaled-score domain, natural log.
  R7 a row with no visible key (unreachable under R2: the diagonal is always
     visible) is defined as O = 0, LSE = -inf.

Every part of this module is pinned by tests against closed forms, brute force,
invariants and a library routine; see the test module for the oracle.
"""
from __future__ import annotations

import numpy as np

_NEG_INF = -np.inf


def fp32_scale(scale: float) -> float:
    """R1: the fp64 value of the fp32 number the ABI receives."""
    return float(np.float32(scale))


def visible(rows: np.ndarray, S: int, causal: bool, window: int = 0,
            n_sink: int = 0) -> np.ndarray:
    """Boolean [len(rows), S]: may query row i attend to key j?  (R2-R5)"""
    rows = np.asarray(rows, dtype=np.int64)
    i = rows[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    if not causal:
        if window:
            raise ValueError("a sliding window needs the causal mask")
        return np.ones((rows.size, S), dtype=bool)
    keep = j <= i
    if window > 0:
        in_window = (i - j) < window
        is_sink = j < n_sink
        keep = keep & (in_window | is_sink)
    return keep


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)   # exact for f32 / f16 inputs
    return a


def attention_fwd(q, k, v, *, causal: bool, scale: float, window: int = 0,
                  n_sink: int = 0, rows=None, chunk: int = 1024, return_probs: bool = False):
    """Materialised attention in fp64.

    q, k, v: arrays [B, H, S, D] (any float dtype; upcast exactly to fp64).
    rows: optional 1-D array of query positions to compute (default: all).
    Returns (O [B, H, R, D], LSE [B, H, R]) in fp64, R = len(rows); with
    return_probs=True also the normalised softmax matrix P [B, H, R, S]
    (small inputs only).

    Each query row's full score row over all S keys is formed at once
    (softmax is row-wise, so computing a chunk of rows at a time is the same
    definition; no online rescaling or key tiling happens here).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, S, D = q.shape
    if k.shape != (B, H, S, D) or v.shape != (B, H, S, D):
        raise ValueError("q, k, v must share the shape [B, H, S, D]")
    s = fp32_scale(scale)
    rows = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    O = np.zeros((B, H, rows.size, D))
    LSE = np.full((B, H, rows.size), _NEG_INF)
    P = np.zeros((B, H, rows.size, S)) if return_probs else None
    for c0 in range(0, rows.size, chunk):
        rr = rows[c0:c0 + chunk]
        keep = visible(rr, S, causal, window, n_sink)
        any_visible = keep.any(axis=1)
        for b in range(B):
            for h in range(H):
                scores = (q[b, h, rr, :] @ k[b, h].T) * s          # [rows, S]
                scores = np.where(keep, scores, _NEG_INF)
                m = scores.max(axis=1)
                m_safe = np.where(any_visible, m, 0.0)
                p = np.exp(scores - m_safe[:, None])                # masked -> 0
                l = p.sum(axis=1)
                l_safe = np.where(any_visible, l, 1.0)
                O[b, h, c0:c0 + rr.size] = (p @ v[b, h]) / l_safe[:, None]
                LSE[b, h, c0:c0 + rr.size] = np.where(any_visible, m + np.log(l_safe),
                                                      _NEG_INF)
                if return_probs:
                    P[b, h, c0:c0 + rr.size] = p / l_safe[:, None]
    if return_probs:
        return O, LSE, P
    return O, LSE


def attention_flops(B: int, H: int, S: int, D: int, causal: bool) -> float:
    """Nominal work of the two contractions: 4*B*H*S^2*D, halved under the causal mask."""
    f = 4.0 * B * H * S * S * D
    return f / 2.0 if causal else f


def visible_pairs(S: int, causal: bool, window: int = 0, n_sink: int = 0) -> int:
    """Number of (query, key) pairs the mask keeps for one head, counted row by row."""
    total = 0
    for c0 in range(0, S, 2048):
        rr = np.arange(c0, min(S, c0 + 2048))
        total += int(visible(rr, S, causal, window, n_sink).sum())
    return total
