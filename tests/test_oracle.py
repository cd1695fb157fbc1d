"""Pins for the fp64 oracle, CPU only.

Each pin checks the oracle against something other than itself: brute force
over scalar loops, a closed form, an invariant, a special case that reduces to
a library routine, the Lab 3 page's worked example, or the tiled CPU model at
several block sizes. Every pin is a function of the oracle module, so the
mutation test at the bottom can feed it oracles with planted mistakes and check
that each mistake is caught by at least one pin.
"""
from __future__ import annotations

import importlib.util
import json
import math
import os
import pathlib
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import fa_inputs
import oracle
from oracle import attention as ORACLE
from tiled_model import tiled_attention

GOLDEN = pathlib.Path(__file__).parent / "golden"

# (causal, window, n_sink)
MASKS = [(False, 0, 0), (True, 0, 0), (True, 3, 0), (True, 3, 2), (True, 5, 1), (True, 1, 0),
         (True, 1, 3)]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _qkv(B, H, S, D, seed):
    return (_rand((B, H, S, D), seed), _rand((B, H, S, D), seed + 1),
            _rand((B, H, S, D), seed + 2))


# --------------------------------------------------------------------------- #
# Pins. Each takes the oracle module and raises AssertionError on a mismatch.
# --------------------------------------------------------------------------- #

def _brute(q, k, v, causal, scale, window, n_sink):
    """Scalar loops over every (b, h, i, j, d) with math.fsum/exp/log."""
    s = float(np.float32(scale))
    B, H, S, D = q.shape
    O = np.zeros((B, H, S, D))
    L = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            for i in range(S):
                keys = []
                for j in range(S):
                    if causal:
                        if j > i:
                            continue
                        if window > 0 and i - j >= window and j >= n_sink:
                            continue
                    keys.append(j)
                sc = [s * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) for j in keys]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = math.fsum(e)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(e[t] * v[b, h, j, d] for t, j in enumerate(keys)) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


def pin_bruteforce(orc):
    cases = [(2, 2, 11, 5, 0.37), (1, 2, 12, 8, 0.125), (1, 1, 7, 3, 1.0), (2, 1, 9, 4, 60.0)]
    for ci, (B, H, S, D, sc) in enumerate(cases):
        q, k, v = _qkv(B, H, S, D, 10 + ci)
        for causal, w, ns in MASKS:
            O, L = orc.attention_fwd(q, k, v, causal=causal, scale=sc, window=w, n_sink=ns)
            Ob, Lb = _brute(q, k, v, causal, sc, w, ns)
            tol = 1e-12 * max(1.0, sc)
            assert np.allclose(O, Ob, rtol=0, atol=tol), (ci, causal, w, ns, np.abs(O - Ob).max())
            assert np.allclose(L, Lb, rtol=tol, atol=tol), (ci, causal, w, ns)


def pin_probs(orc):
    q, k, v = _qkv(2, 2, 17, 6, 3)
    for causal, w, ns in MASKS:
        O, L, P = orc.attention_fwd(q, k, v, causal=causal, scale=0.4, window=w, n_sink=ns,
                                   return_probs=True)
        assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
        assert (P >= 0).all()
        # masked pairs get exactly zero weight: P = 0 above the diagonal
        if causal:
            assert (np.triu(P[0, 0], k=1) == 0).all()
        assert np.allclose(np.einsum("bhij,bhjd->bhid", P, v), O, rtol=0, atol=1e-12)


def pin_constant_v(orc):
    q, k, _ = _qkv(1, 3, 20, 4, 5)
    c = np.array([1.5, -2.25, 0.0, 3.0])
    v = np.broadcast_to(c, (1, 3, 20, 4)).copy()
    for causal, w, ns in MASKS:
        O, _ = orc.attention_fwd(q, k, v, causal=causal, scale=0.7, window=w, n_sink=ns)
        assert np.allclose(O, c, rtol=0, atol=1e-12)


def pin_causal_row0(orc):
    q, k, v = _qkv(2, 2, 16, 8, 7)
    for w, ns in [(0, 0), (4, 0), (4, 3), (1, 5)]:
        O, L = orc.attention_fwd(q, k, v, causal=True, scale=0.3, window=w, n_sink=ns)
        assert np.array_equal(O[:, :, 0], v[:, :, 0])       # P = [1]: bit-exact
        s = float(np.float32(0.3))
        lse0 = s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
        assert np.allclose(L[:, :, 0], lse0, rtol=1e-15, atol=1e-15)


def pin_prefix_independence(orc):
    B, H, S, D, t = 1, 2, 24, 4, 9
    q, k, v = _qkv(B, H, S, D, 11)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rng = np.random.default_rng(99)
    for a in (q2, k2, v2):
        a[:, :, t:] = rng.standard_normal(a[:, :, t:].shape) * 5
    for w, ns in [(0, 0), (5, 0), (5, 2)]:
        O1, L1 = orc.attention_fwd(q, k, v, causal=True, scale=0.5, window=w, n_sink=ns)
        O2, L2 = orc.attention_fwd(q2, k2, v2, causal=True, scale=0.5, window=w, n_sink=ns)
        assert np.array_equal(O1[:, :, :t], O2[:, :, :t])
        assert np.array_equal(L1[:, :, :t], L2[:, :, :t])
        assert not np.array_equal(O1[:, :, t:], O2[:, :, t:])


def pin_tiled_block_invariance(orc):
    """Lab 3, exercise 1: the block size (1, 7, 16, 64, ragged last block)
    must not change the result of the online-softmax loop."""
    for S in (64, 65, 100):
        q, k, v = _qkv(1, 2, S, 8, S)
        for causal, w, ns in [(False, 0, 0), (True, 0, 0), (True, 9, 0), (True, 9, 3),
                              (True, 40, 4)]:
            O, L = orc.attention_fwd(q, k, v, causal=causal, scale=0.35, window=w, n_sink=ns)
            for bs in (1, 7, 16, 64):
                Ot, Lt = tiled_attention(q, k, v, causal=causal, scale=float(np.float32(0.35)),
                                         window=w, n_sink=ns, bs=bs)
                assert np.allclose(O, Ot, rtol=0, atol=1e-12), (S, causal, w, ns, bs)
                assert np.allclose(L, Lt, rtol=0, atol=1e-12), (S, causal, w, ns, bs)


def pin_lab3_worked_example(orc):
    g = json.loads((GOLDEN / "lab3_worked_example.json").read_text())
    Q, K, V = fa_inputs.lab3_example()
    q, k, v = (a.reshape(1, 1, g["n"], g["d"]) for a in (Q, K, V))
    scale = 1.0 / math.sqrt(g["d"])           # 0.25, exact in fp32
    O, L = orc.attention_fwd(q, k, v, causal=True, scale=scale)
    cnt = {}
    Ot, Lt = tiled_attention(q, k, v, causal=True, scale=scale, bs=g["block_size"], counter=cnt)
    assert np.abs(O - Ot).max() <= g["bound_used_in_tests"]
    assert np.abs(L - Lt).max() <= g["bound_used_in_tests"]


def pin_sdpa_library(orc):
    """Special case that reduces to a library routine: torch's scaled dot-product
    attention on the CPU in fp64 with a boolean mask; LSE against torch.logsumexp."""
    q, k, v = _qkv(2, 3, 33, 16, 21)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    for causal, w, ns in MASKS + [(True, 8, 4), (True, 40, 0)]:
        sc = 1.0 / math.sqrt(13.0)
        s = float(np.float32(sc))
        O, L = orc.attention_fwd(q, k, v, causal=causal, scale=sc, window=w, n_sink=ns)
        i = torch.arange(33)[:, None]
        j = torch.arange(33)[None, :]
        if causal:
            mask = j <= i
            if w:
                mask = mask & (((i - j) < w) | (j < ns))
        else:
            mask = torch.ones(33, 33, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s)
        assert np.allclose(O, ref.numpy(), rtol=0, atol=1e-12), (causal, w, ns)
        scores = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * s
        scores = scores.masked_fill(~mask, float("-inf"))
        assert np.allclose(L, torch.logsumexp(scores, dim=-1).numpy(), rtol=0, atol=1e-12)


def _count_closed_form(i, S, causal, W, n_sink):
    if not causal:
        return S
    if W == 0:
        return i + 1
    return min(i + 1, W) + min(n_sink, max(0, i - W + 1))


def pin_closed_form_scale0(orc):
    """scale = 0 makes every visible key weigh the same: O_i is the mean of the
    visible V rows and LSE_i = ln |A(i)|, with |A(i)| counted in closed form."""
    S = 40
    q, k, v = _qkv(1, 1, S, 6, 31)
    for causal, w, ns in MASKS + [(True, 10, 4), (True, 10, 12), (True, 64, 2)]:
        O, L = orc.attention_fwd(q, k, v, causal=causal, scale=0.0, window=w, n_sink=ns)
        for i in range(S):
            n = _count_closed_form(i, S, causal, w, ns)
            assert abs(L[0, 0, i] - math.log(n)) <= 1e-12, (causal, w, ns, i)
            # keys: most recent min(i+1, W) plus the sinks outside the window
            if not causal:
                keys = list(range(S))
            else:
                lo = 0 if w == 0 else max(0, i - w + 1)
                keys = list(range(lo, i + 1)) + list(range(0, min(ns, lo) if w else 0))
            assert len(keys) == n
            assert np.allclose(O[0, 0, i], v[0, 0, keys].mean(axis=0), rtol=0, atol=1e-12)


def pin_window_degenerate(orc):
    S = 21
    q, k, v = _qkv(2, 2, S, 5, 41)
    Oc, Lc = orc.attention_fwd(q, k, v, causal=True, scale=0.6)
    for w in (S, S + 5, 1000):
        Ow, Lw = orc.attention_fwd(q, k, v, causal=True, scale=0.6, window=w, n_sink=3)
        assert np.array_equal(Oc, Ow) and np.array_equal(Lc, Lw)
    O1, L1 = orc.attention_fwd(q, k, v, causal=True, scale=0.6, window=1)
    assert np.array_equal(O1, v)
    s = float(np.float32(0.6))
    assert np.allclose(L1, s * np.einsum("bhsd,bhsd->bhs", q, k), rtol=1e-15, atol=1e-15)
    q1, k1, v1 = q[:, :, :1], k[:, :, :1], v[:, :, :1]
    O2, _ = orc.attention_fwd(q1, k1, v1, causal=False, scale=0.6)
    assert np.array_equal(O2, v1)


def pin_shift_invariance(orc):
    q, k, v = _qkv(1, 2, 30, 7, 51)
    c = np.random.default_rng(5).standard_normal(7) * 3
    s = float(np.float32(0.45))
    for causal, w, ns in MASKS:
        O, L = orc.attention_fwd(q, k, v, causal=causal, scale=0.45, window=w, n_sink=ns)
        O2, L2 = orc.attention_fwd(q, k + c, v, causal=causal, scale=0.45, window=w, n_sink=ns)
        assert np.allclose(O, O2, rtol=0, atol=1e-12)
        assert np.allclose(L2, L + s * (q @ c), rtol=0, atol=1e-12)


def pin_permutation_noncausal(orc):
    q, k, v = _qkv(1, 2, 25, 6, 61)
    rng = np.random.default_rng(7)
    pk = rng.permutation(25)
    pq = rng.permutation(25)
    O, L = orc.attention_fwd(q, k, v, causal=False, scale=0.5)
    O2, L2 = orc.attention_fwd(q[:, :, pq], k[:, :, pk], v[:, :, pk], causal=False, scale=0.5)
    assert np.allclose(O2, O[:, :, pq], rtol=0, atol=1e-12)
    assert np.allclose(L2, L[:, :, pq], rtol=0, atol=1e-12)


def pin_row_subset(orc):
    """Computing a subset of query rows gives the same rows as the full call."""
    q, k, v = _qkv(2, 2, 50, 8, 71)
    rows = np.array([0, 3, 17, 49, 25])
    for causal, w, ns in MASKS:
        O, L = orc.attention_fwd(q, k, v, causal=causal, scale=0.3, window=w, n_sink=ns)
        Os, Ls = orc.attention_fwd(q, k, v, causal=causal, scale=0.3, window=w, n_sink=ns,
                                   rows=rows, chunk=2)
        assert np.array_equal(Os, O[:, :, rows]) or np.allclose(Os, O[:, :, rows], rtol=0,
                                                                 atol=1e-15)
        assert np.allclose(Ls, L[:, :, rows], rtol=0, atol=1e-15)


PINS = [pin_bruteforce, pin_probs, pin_constant_v, pin_causal_row0, pin_prefix_independence,
        pin_tiled_block_invariance, pin_lab3_worked_example, pin_sdpa_library,
        pin_closed_form_scale0, pin_window_degenerate, pin_shift_invariance,
        pin_permutation_noncausal, pin_row_subset]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(ORACLE)


# --------------------------------------------------------------------------- #
# Other page-fixed facts
# --------------------------------------------------------------------------- #

def test_lab3_block_pair_count():
    """Lab 3, exercise 3: with n=64 and blocks of 16 the causal loop visits 10 of
    the 16 block pairs, nb(nb+1)/2 of nb^2."""
    g = json.loads((GOLDEN / "lab3_worked_example.json").read_text())
    Q, K, V = fa_inputs.lab3_example()
    q, k, v = (a.reshape(1, 1, 64, 16) for a in (Q, K, V))
    cnt = {}
    tiled_attention(q, k, v, causal=True, scale=0.25, bs=16, counter=cnt)
    assert cnt["visited_pairs"] == g["exercise_3_visited_block_pairs"]
    assert cnt["all_pairs"] == g["exercise_3_all_block_pairs"]
    assert g["n"] ** 2 == g["exercise_2_score_entries_full"]
    assert g["block_size"] ** 2 == g["exercise_2_score_entries_per_block"]


def test_tiled_block_guide_example():
    """The NumPy tiled-block guide's validation case (non-causal, N=512, d=64,
    tile 128, seed 42, fp32 inputs) agrees within the bound it asserts."""
    g = json.loads((GOLDEN / "tiled_block_guide.json").read_text())
    rng = np.random.default_rng(42)
    Q, K, V = (rng.normal(size=(g["N"], g["d"])).astype(np.float32) for _ in range(3))
    q, k, v = (a.astype(np.float64).reshape(1, 1, g["N"], g["d"]) for a in (Q, K, V))
    O, _ = ORACLE.attention_fwd(q, k, v, causal=False, scale=1 / math.sqrt(g["d"]))
    Ot, _ = tiled_attention(q, k, v, causal=False, scale=float(np.float32(1 / 8)),
                            bs=g["tile_size"])
    assert np.abs(O - Ot).max() < g["asserted_bound_max_abs_difference"]
    assert np.abs(O - Ot).max() < 1e-12


def test_visible_pair_counts():
    """Kept (query, key) pairs per head, used for the FLOP accounting, against
    their closed forms."""
    S = 4096
    assert ORACLE.visible_pairs(S, True) == S * (S + 1) // 2 == 8390656
    S, W, ns = 8192, 1024, 4
    closed = W * (W + 1) // 2 + (S - W) * W + sum(min(ns, i - W + 1) for i in range(W, S))
    assert ORACLE.visible_pairs(S, True, W, ns) == closed == 7893498
    assert ORACLE.visible_pairs(1024, False) == 1024 * 1024
    assert ORACLE.attention_flops(4, 16, 4096, 128, True) == 4 * 4 * 16 * 4096 ** 2 * 128 / 2


def test_window_without_causal_rejected():
    with pytest.raises(ValueError):
        ORACLE.visible(np.arange(4), 4, causal=False, window=2)


def test_generator_is_seeded_and_rounded():
    a = fa_inputs.make_qkv(1, 2, 8, 16, "bf16", seed=3)
    b = fa_inputs.make_qkv(1, 2, 8, 16, "bf16", seed=3)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    # the Lab 3 draw: fp64 N(0,1) from default_rng(0), then fp32
    q, k, v = fa_inputs.make_workload(fa_inputs.WORKLOADS["causal_b1h1s64d16_f32"])
    Q, K, V = fa_inputs.lab3_example()
    assert np.array_equal(fa_inputs.to_f64(q)[0, 0], Q.astype(np.float32).astype(np.float64))
    assert np.array_equal(fa_inputs.to_f64(v)[0, 0], V.astype(np.float32).astype(np.float64))


# --------------------------------------------------------------------------- #
# Planted mistakes: every plausible slip in the oracle must fail some pin.
# --------------------------------------------------------------------------- #

MUTATIONS = {
    "causal_strict": ("keep = j <= i", "keep = j < i"),
    "causal_flipped": ("keep = j <= i", "keep = j >= i"),
    "window_off_by_one": ("in_window = (i - j) < window", "in_window = (i - j) <= window"),
    "sinks_dropped": ("keep = keep & (in_window | is_sink)", "keep = keep & in_window"),
    "sinks_ignore_causality": ("keep = keep & (in_window | is_sink)",
                               "keep = (keep & in_window) | is_sink"),
    "scale_dropped": ("@ k[b, h].T) * s ", "@ k[b, h].T) "),
    "scale_not_fp32": ("return float(np.float32(scale))", "return float(scale)"),
    "operands_swapped": ("(q[b, h, rr, :] @ k[b, h].T)", "(k[b, h, rr, :] @ q[b, h].T)"),
    "no_normalisation": ("(p @ v[b, h]) / l_safe[:, None]", "(p @ v[b, h])"),
    "lse_log2": ("m + np.log(l_safe)", "m + np.log2(l_safe)"),
    "lse_without_max": ("m + np.log(l_safe)", "np.log(l_safe)"),
    "no_max_subtraction": ("p = np.exp(scores - m_safe[:, None])", "p = np.exp(scores)"),
    "v_rows_misaligned": ("(p @ v[b, h])", "(p @ np.roll(v[b, h], 1, axis=0))"),
}


def _mutant(name):
    src = pathlib.Path(ORACLE.__file__).read_text()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, name
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                caught.append(pin.__name__)
    assert caught, f"mutation {name} passes every pin"
