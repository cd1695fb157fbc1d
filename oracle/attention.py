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
  R8 grouped K/V heads (Lesson 91 deck, slide 32 "MQA: one shared K, V for all
     query heads"): with Hq query heads and Hkv key/value heads (Hkv divides
     Hq), query head h reads key/value head h // (Hq / Hkv), i.e. consecutive
     query heads form the groups. Hkv = 1 is MQA, Hkv = Hq ordinary attention.
  R10 split keys (the tiled-block guide's closing note on reducing partial
     outputs across workers): attention restricted to a key range [kb, ke)
     gives a partial (O_r, LSE_r) -- O_r normalised within the range, and
     (O_r, LSE_r) = (0, -inf) for a row that sees no key there; partials of
     disjoint ranges covering all keys merge into the full result by
     LSE = log sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r.
  R9 ALiBi (Lesson 91 deck, slides 20-25): the logit of (i, j) in head h gains
     the bias -m_h * |i - j| before the softmax, on top of the scaled score;
     the slopes are inputs (fp32, rounded first like the scale), and
     alibi_slopes(H) gives the deck's geometric rule m_h = 2^(-8h/H), h = 1..H.

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


def alibi_slopes(H: int) -> np.ndarray:
    """R9: the deck's slope rule, m_h = 2^(-8h/H) for heads h = 1..H (slide 23)."""
    return np.array([2.0 ** (-8.0 * h / H) for h in range(1, H + 1)])


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """R8: the key/value head that query head h reads."""
    return h // (Hq // Hkv)


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)   # exact for f32 / f16 inputs
    return a


def attention_fwd(q, k, v, *, causal: bool, scale: float, window: int = 0,
                  n_sink: int = 0, rows=None, chunk: int = 1024, return_probs: bool = False,
                  alibi_slopes=None, key_range=None):
    """Materialised attention in fp64.

    q: [B, Hq, S, D]; k, v: [B, Hkv, S, D] with Hkv dividing Hq (R8); any float
    dtype, upcast exactly to fp64. alibi_slopes: optional [Hq] slopes (R9).
    key_range: optional (kb, ke) -- only keys kb <= j < ke are visible (R10).
    rows: optional 1-D array of query positions to compute (default: all).
    Returns (O [B, Hq, R, D], LSE [B, Hq, R]) in fp64, R = len(rows); with
    return_probs=True also the normalised softmax matrix P [B, Hq, R, S]
    (small inputs only).

    Each query row's full score row over all S keys is formed at once
    (softmax is row-wise, so computing a chunk of rows at a time is the same
    definition; no online rescaling or key tiling happens here).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, S, D = q.shape
    Hkv = k.shape[1] if k.ndim == 4 else 0
    if Hkv < 1 or k.shape != (B, Hkv, S, D) or v.shape != (B, Hkv, S, D) or H % Hkv:
        raise ValueError("k, v must be [B, Hkv, S, D] with Hkv dividing the query heads")
    s = fp32_scale(scale)
    slopes = None
    if alibi_slopes is not None:
        slopes = np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64)
        if slopes.shape != (H,):
            raise ValueError("alibi_slopes must hold one slope per query head")
    rows = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    j_idx = np.arange(S, dtype=np.int64)[None, :]
    O = np.zeros((B, H, rows.size, D))
    LSE = np.full((B, H, rows.size), _NEG_INF)
    P = np.zeros((B, H, rows.size, S)) if return_probs else None
    for c0 in range(0, rows.size, chunk):
        rr = rows[c0:c0 + chunk]
        keep = visible(rr, S, causal, window, n_sink)
        if key_range is not None:
            keep = keep & (j_idx >= key_range[0]) & (j_idx < key_range[1])
        any_visible = keep.any(axis=1)
        dist = np.abs(rr[:, None] - j_idx).astype(np.float64)
        for b in range(B):
            for h in range(H):
                g = kv_head(h, H, Hkv)
                scores = (q[b, h, rr, :] @ k[b, g].T) * s          # [rows, S]
                if slopes is not None:
                    scores = scores - slopes[h] * dist
                scores = np.where(keep, scores, _NEG_INF)
                m = scores.max(axis=1)
                m_safe = np.where(any_visible, m, 0.0)
                p = np.exp(scores - m_safe[:, None])                # masked -> 0
                l = p.sum(axis=1)
                l_safe = np.where(any_visible, l, 1.0)
                O[b, h, c0:c0 + rr.size] = (p @ v[b, g]) / l_safe[:, None]
                LSE[b, h, c0:c0 + rr.size] = np.where(any_visible, m + np.log(l_safe),
                                                      _NEG_INF)
                if return_probs:
                    P[b, h, c0:c0 + rr.size] = p / l_safe[:, None]
    if return_probs:
        return O, LSE, P
    return O, LSE


def attention_bwd(q, k, v, dO, *, causal: bool, scale: float, window: int = 0,
                  n_sink: int = 0, alibi_slopes=None, chunk: int = 1024):
    """Gradients of O = softmax(Q K^T * scale + bias + mask) V by definition, fp64.

    q, dO: [B, Hq, S, D]; k, v: [B, Hkv, S, D] (R8). Returns (dQ, dK, dV) in fp64
    with the shapes of q, k, v; dK, dV of a key/value head sum over the query
    heads that read it. With P the softmax matrix of a head (rows sum to 1 over
    the visible keys) and dP = dO V^T:
        dV = P^T dO,   dS = P * (dP - rowsum(P * dP)),
        dQ = scale * dS K,   dK = scale * dS^T Q.
    (rowsum(P * dP) = rowsum(dO * O): the derivative of a softmax row.) The
    ALiBi bias and the mask are constants, so they only enter through P.
    Backward by recomputation, as the Lesson 91 deck's closing note describes
    it: nothing of the forward pass but its inputs (and LSE) is kept.
    """
    q, k, v, dO = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dO)
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or dO.shape != q.shape or H % Hkv:
        raise ValueError("q, dO: [B, H, S, D]; k, v: [B, H_kv, S, D] with H_kv dividing H")
    s = fp32_scale(scale)
    slopes = None if alibi_slopes is None else \
        np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    j_idx = np.arange(S, dtype=np.int64)[None, :]
    for c0 in range(0, S, chunk):
        rr = np.arange(c0, min(S, c0 + chunk), dtype=np.int64)
        keep = visible(rr, S, causal, window, n_sink)
        dist = np.abs(rr[:, None] - j_idx).astype(np.float64)
        for b in range(B):
            for h in range(H):
                g = kv_head(h, H, Hkv)
                scores = (q[b, h, rr, :] @ k[b, g].T) * s
                if slopes is not None:
                    scores = scores - slopes[h] * dist
                scores = np.where(keep, scores, _NEG_INF)
                m = scores.max(axis=1)
                m_safe = np.where(np.isfinite(m), m, 0.0)
                p = np.exp(scores - m_safe[:, None])
                l = p.sum(axis=1)
                P = p / np.where(l > 0, l, 1.0)[:, None]            # [rows, S]
                dP = dO[b, h, rr, :] @ v[b, g].T                     # [rows, S]
                dS = P * (dP - (P * dP).sum(axis=1)[:, None])
                dv[b, g] += P.T @ dO[b, h, rr, :]
                dq[b, h, rr, :] = s * (dS @ k[b, g])
                dk[b, g] += s * (dS.T @ q[b, h, rr, :])
    return dq, dk, dv


def merge_partials(O_parts, LSE_parts):
    """R10: merge partial results of disjoint key ranges.

    O_parts: [R, ..., D] (partial outputs, each normalised within its range);
    LSE_parts: [R, ...]. Returns (O [..., D], LSE [...]). Parts with LSE = -inf
    contribute nothing; if every part is -inf the row is (0, -inf).
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    L = np.asarray(LSE_parts, dtype=np.float64)
    m = L.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(L - m_safe)                      # -inf parts -> 0
    tot = w.sum(axis=0)
    tot_safe = np.where(tot > 0, tot, 1.0)
    LSE = np.where(tot > 0, m_safe + np.log(tot_safe), _NEG_INF)
    O = (w[..., None] * O_parts).sum(axis=0) / tot_safe[..., None]
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
