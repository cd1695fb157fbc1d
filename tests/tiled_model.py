"""CPU model of the tiled online-softmax forward pass, fp64 -- test helper.

The tiled method keeps, for each query row, three numbers per stretch of keys
it has seen: the largest score m, the sum of exponentials l taken against m,
and the numerator vector n (the exponential-weighted sum of value rows, also
against m). The update equations of the Lesson 91 deck (slide 11, "Online
softmax: tiled update equations") say how two such summaries combine when the
running max moves: both are brought to the larger max by the factor
exp(m_old - m_new) and added. Written as an operation on summaries,

    (m, l, n) + (m', l', n') = (M, l e^(m - M) + l' e^(m' - M), n e^(m - M) + n' e^(m' - M)),
    M = max(m, m'),

it is associative, with (-inf, 0, 0) as the neutral element, and the
attention output of a row is n / l of the combination of all its key blocks,
its logsumexp m + ln l. This model builds each (query block, key block) pair's
summary from that block's scores alone and folds the summaries of a query
block's key blocks left to right, which is the order in which the tiled loop of
the Lab 3 page ("Tiled attention with online softmax") visits them; `fold` can
also combine them in a balanced tree, which must give the same result.

Beyond the pages' single head and causal mask it handles several heads, the
sliding window and the sink keys, and summaries of blocks in which a row sees
no key (those are the neutral element). Its only role is to pin the oracle:
for any block size (1, 7, 16, 64; ragged last block) it must reproduce the
oracle's materialised result, the invariance the Lab 3 page's first exercise
asks about.
"""
from __future__ import annotations

import numpy as np


def _visible(i0, i1, j0, j1, causal, window, n_sink):
    i = np.arange(i0, i1)[:, None]
    j = np.arange(j0, j1)[None, :]
    if not causal:
        return np.ones((i1 - i0, j1 - j0), dtype=bool)
    ok = j <= i
    if window:
        ok &= ((i - j) < window) | (j < n_sink)
    return ok


class Summary:
    """(m, l, n) of a set of keys, per query row of a block: m [R], l [R], n [R, D]."""

    def __init__(self, m, l, n):
        self.m, self.l, self.n = m, l, n

    @staticmethod
    def empty(rows, D, dtype=np.float64):
        return Summary(np.full(rows, -np.inf, dtype), np.zeros(rows, dtype),
                       np.zeros((rows, D), dtype))

    @staticmethod
    def of_block(scores, visible, v_block):
        """The summary of one key block from its scores [R, C], visibility
        [R, C] and value rows [C, D]; a row with no visible key is empty."""
        s = np.where(visible, scores, -np.inf)
        m = s.max(axis=1)
        seen = np.isfinite(m)
        w = np.zeros_like(s)
        w[seen] = np.exp(s[seen] - m[seen, None])
        return Summary(m, w.sum(axis=1), w @ v_block)

    def __add__(self, other):
        M = np.maximum(self.m, other.m)
        finite = np.isfinite(M)
        a = np.zeros_like(M)
        b = np.zeros_like(M)
        a[finite] = np.exp(self.m[finite] - M[finite])     # empty side -> factor 0
        b[finite] = np.exp(other.m[finite] - M[finite])
        return Summary(M, self.l * a + other.l * b, self.n * a[:, None] + other.n * b[:, None])

    def output(self):
        """(O rows, LSE rows); rows that saw nothing stay (0, -inf)."""
        seen = self.l > 0
        O = np.zeros_like(self.n)
        O[seen] = self.n[seen] / self.l[seen, None]
        LSE = np.full(self.m.shape, -np.inf)
        LSE[seen] = self.m[seen] + np.log(self.l[seen])
        return O, LSE


def fold(summaries, order="left", rows=0, D=0, dtype=np.float64):
    """Combine summaries left to right (the tiled loop's order) or as a
    balanced tree; an empty list gives the neutral element."""
    if not summaries:
        return Summary.empty(rows, D, dtype)
    if order == "left":
        acc = summaries[0]
        for s in summaries[1:]:
            acc = acc + s
        return acc
    level = list(summaries)
    while len(level) > 1:
        level = [level[i] + level[i + 1] if i + 1 < len(level) else level[i]
                 for i in range(0, len(level), 2)]
    return level[0]


def tiled_attention(q, k, v, *, causal, scale, window=0, n_sink=0, bs=16, counter=None,
                    order="left"):
    """q, k, v [B, H, S, D], fp64 (or fp16 for the precision study: every
    step then runs in the inputs' dtype). Returns (O, LSE). `counter` (a dict)
    receives the number of (query block, key block) pairs whose block holds a
    visible key, and the number of all pairs, for the first head."""
    B, H, S, D = q.shape
    O = np.zeros_like(q)
    LSE = np.zeros(q.shape[:3], q.dtype)
    scale = q.dtype.type(scale)
    visited = 0
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, h], k[b, h], v[b, h]
            for i0 in range(0, S, bs):
                i1 = min(i0 + bs, S)
                parts = []
                for j0 in range(0, S, bs):
                    j1 = min(j0 + bs, S)
                    vis = _visible(i0, i1, j0, j1, causal, window, n_sink)
                    if not vis.any():
                        continue            # a block the mask hides is never formed
                    if b == 0 and h == 0:
                        visited += 1
                    parts.append(Summary.of_block((Q[i0:i1] @ K[j0:j1].T) * scale, vis,
                                                  V[j0:j1]))
                O[b, h, i0:i1], LSE[b, h, i0:i1] = fold(parts, order, i1 - i0, D,
                                                         q.dtype).output()
    if counter is not None:
        nb = -(-S // bs)
        counter["visited_pairs"] = visited
        counter["all_pairs"] = nb * nb
    return O, LSE
