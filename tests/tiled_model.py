"""CPU model of the tiled online-softmax forward pass, fp64 -- test helper.

It follows the algorithm of the Lab 3 page ("Tiled attention with online
softmax", its `tiled` function) and the update equations of the Lesson 91 deck
(slide 11, "Online softmax: tiled update equations"): for each query block, a
running max m, running denominator l and running numerator o are carried over
key blocks; each new block rescales what was accumulated by exp(m_old - m_new)
before adding its own exp(s - m_new) terms; the output o / l is written once.

Generalised here (and nowhere else) to several heads, the sliding window and
the sink keys, and to rows whose first visited key block is fully masked (for
those, the update uses 0 in place of an -inf running max so that no
(-inf) - (-inf) is ever formed). Its only role is to pin the oracle: for any
block size (1, 7, 16, 64; ragged last block) it must reproduce the oracle's
materialised result, which is the invariance the Lab 3 page's first exercise
asks about.
"""
from __future__ import annotations

import numpy as np


def _keep(i0, i1, j0, j1, causal, window, n_sink):
    i = np.arange(i0, i1)[:, None]
    j = np.arange(j0, j1)[None, :]
    if not causal:
        return np.ones((i1 - i0, j1 - j0), dtype=bool)
    ok = j <= i
    if window:
        ok &= ((i - j) < window) | (j < n_sink)
    return ok


def tiled_attention(q, k, v, *, causal, scale, window=0, n_sink=0, bs=16, counter=None):
    """q, k, v fp64 [B, H, S, D]. Returns (O, LSE). `counter` (a dict) receives
    the number of key blocks visited and the number of (q-block, k-block) pairs."""
    B, H, S, D = q.shape
    O = np.zeros_like(q)
    LSE = np.zeros(q.shape[:3])
    visited = 0
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, h], k[b, h], v[b, h]
            for i0 in range(0, S, bs):
                i1 = min(i0 + bs, S)
                qb = Q[i0:i1]
                m = np.full(i1 - i0, -np.inf)
                l = np.zeros(i1 - i0)
                o = np.zeros((i1 - i0, D))
                # Causal: only key blocks that start at or before the last row of
                # this query block can hold a visible key.
                j_end = i1 if causal else S
                for j0 in range(0, j_end, bs):
                    j1 = min(j0 + bs, S)
                    keep = _keep(i0, i1, j0, j1, causal, window, n_sink)
                    if not keep.any():
                        continue            # a fully masked block adds nothing
                    if b == 0 and h == 0:
                        visited += 1
                    s = (qb @ K[j0:j1].T) * scale
                    s = np.where(keep, s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    m_use = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.exp(m - m_use)          # exp(-inf) = 0 on the first block
                    p = np.exp(s - m_use[:, None])
                    l = l * alpha + p.sum(axis=1)
                    o = o * alpha[:, None] + p @ V[j0:j1]
                    m = m_new
                O[b, h, i0:i1] = o / l[:, None]
                LSE[b, h, i0:i1] = m + np.log(l)
    if counter is not None:
        nb = -(-S // bs)
        counter["visited_pairs"] = visited
        counter["all_pairs"] = nb * nb
    return O, LSE
