"""GPU parity: the gfx950 kernels through the C ABI against the fp64 oracle.

Inputs are seeded (fa_inputs); the oracle reads the very values stored on the
GPU (exactly upcast to fp64) and its output is not rounded before comparison.
Bars: max |dO| <= 1e-5 (f32), 4e-3 (f16), 1.6e-2 (bf16); |dLSE| <= 1e-3 *
max(1, |LSE|).
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import io_aware_tiled_flash_amd as fa
from oracle import attention as ORACLE

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "f16": 4e-3, "bf16": 1.6e-2}
TOL_LSE_REL = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def gpu_fwd(q, k, v, **kw):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.flash_attn_fwd(qd, kd, vd, **kw)
    torch.cuda.synchronize()
    return o, lse


def compare(o, lse, q, k, v, dtype, *, causal, scale, window=0, n_sink=0, heads=None,
            rows=None, label="", tol_o=None, alibi=None):
    """o, lse: GPU results (device tensors). heads: list of (b, h) to check
    (default all); rows: query rows to check (default all). k, v may hold fewer
    heads than q (grouped heads); alibi: optional per-head slopes (numpy)."""
    tol_o = TOL_O[dtype] if tol_o is None else tol_o
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst_o, worst_l = 0.0, 0.0
    for b, h in heads:
        g = ORACLE.kv_head(h, H, Hkv)
        q64 = fa_inputs.to_f64(q[b:b + 1, h:h + 1])
        k64, v64 = (fa_inputs.to_f64(t[b:b + 1, g:g + 1]) for t in (k, v))
        O, L = ORACLE.attention_fwd(q64, k64, v64, causal=causal, scale=scale, window=window,
                                    n_sink=n_sink, rows=rows,
                                    alibi_slopes=None if alibi is None else alibi[h:h + 1])
        r = slice(None) if rows is None else torch.as_tensor(np.asarray(rows))
        og = o[b, h].float().cpu()[r].double().numpy()
        lg = lse[b, h].cpu()[r].double().numpy()
        assert np.isfinite(og).all() and np.isfinite(lg).all(), label
        worst_o = max(worst_o, float(np.abs(og - O[0, 0]).max()))
        worst_l = max(worst_l, float((np.abs(lg - L[0, 0]) / np.maximum(1.0, np.abs(L[0, 0]))).max()))
    _say(f"  {label}: max|dO|={worst_o:.3e} (tol {tol_o:g})  max rel dLSE={worst_l:.3e}")
    if os.environ.get("FA_PARITY_LOG"):
        with open(os.environ["FA_PARITY_LOG"], "a") as f:
            f.write(f"{label}\t{worst_o:.3e}\t{tol_o:g}\t{worst_l:.3e}\n")
    assert worst_o <= tol_o, (label, worst_o)
    assert worst_l <= TOL_LSE_REL, (label, worst_l)
    return worst_o, worst_l


# --------------------------------------------------------------------------- #
# The five workloads
# --------------------------------------------------------------------------- #

def _sample_rows(S, rng, n=192):
    edges = [0, 1, 2, 63, 64, 65, 127, 128, 129, S // 2, S - 129, S - 128, S - 65, S - 64,
             S - 2, S - 1]
    rows = set(r for r in edges if 0 <= r < S)
    rows |= set(rng.choice(S, size=min(n, S), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", [n for n, w in fa_inputs.ALL_WORKLOADS.items() if not w.backward])
def test_workload_parity(name):
    w = fa_inputs.ALL_WORKLOADS[name]
    _say(f"workload {name}: generating inputs")
    q, k, v = fa_inputs.make_workload(w)
    slopes = ORACLE.alibi_slopes(w.H).astype(np.float32) if w.alibi else None
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()
    _say(f"workload {name}: launching")
    if w.n_split > 1:
        o, lse = fa.flash_attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), n_split=w.n_split,
                                         causal=w.causal, window=w.window, n_sink=w.n_sink,
                                         scale=w.scale, alibi_slopes=sd)
        torch.cuda.synchronize()
    else:
        o, lse = gpu_fwd(q, k, v, causal=w.causal, window=w.window, n_sink=w.n_sink,
                         scale=w.scale, alibi_slopes=sd)
    assert o.shape == q.shape and o.dtype == q.dtype and lse.shape == q.shape[:3]
    al = None if slopes is None else slopes.astype(np.float64)
    small = w.B * w.H * w.S <= 32768
    if name == fa_inputs.HEADLINE:
        # every head and row of the headline shape, the oracle on a pool of
        # single-threaded processes (the same code as the bench line's parity)
        import bench
        _say(f"workload {name}: oracle on all {w.B * w.H} heads")
        _, heads, res = bench.cpu_baseline(w, q, k, v, w.B * w.H)
        par = bench.parity(w, heads, res, (o, lse))
        _say(f"  {name} (all rows): max|dO|={par['max_abs_dO']:.3e} (tol {par['tol_O']:g})  "
             f"max rel dLSE={par['max_rel_dLSE']:.3e}")
        assert len(heads) == w.B * w.H and par["rows_per_head"] == w.S
        assert par["max_abs_dO"] <= TOL_O[w.dtype] and par["max_rel_dLSE"] <= TOL_LSE_REL, par
    elif small:
        compare(o, lse, q, k, v, w.dtype, causal=w.causal, scale=w.scale, window=w.window,
                n_sink=w.n_sink, label=name, alibi=al)
    else:
        rng = np.random.default_rng(1234)
        heads = [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 3)]
        rows = _sample_rows(w.S, rng)
        compare(o, lse, q, k, v, w.dtype, causal=w.causal, scale=w.scale, window=w.window,
                n_sink=w.n_sink, heads=heads, rows=rows, label=name + " (sampled rows)", alibi=al)
        # properties at full size: every output finite, causal row 0 is V[0] of its K/V head
        assert torch.isfinite(lse).all()
        assert torch.isfinite(o.float()).all()
        if w.causal:
            G = w.H // w.kv_heads
            assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0].repeat_interleave(G, dim=1))


def test_sequence_longer_than_2_to_the_24():
    """S = 2^24 + 77 keys of D = 128 bf16: one head's K is 4.3 GB, beyond a
    32-bit byte count, so every tile load has to address it correctly. With a
    96-key window and 3 sinks each row sees at most 99 keys, so the oracle
    checks sampled rows on a compacted copy of the keys a row sees: the sinks
    followed by its window, with the query last. The mask depends only on
    i - j and on j < n_sink, so that row's visible set and its scores are the
    same as in the long sequence."""
    S, D, W, NS = (1 << 24) + 77, 128, 96, 3
    scale = 1.0 / math.sqrt(D)
    _say("long sequence: generating inputs on the device")
    q, k, v = fa_inputs.make_qkv_device(S, D, "bf16", seed=11, device="cuda")
    _say("long sequence: launching")
    o, lse = fa.flash_attn_fwd(q, k, v, causal=True, window=W, n_sink=NS, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 2, 3, 97, 98, 99, 100, S // 2, S - 2, S - 1, (1 << 24) - 1, 1 << 24,
                       (1 << 23) + 5]) | set(rng.integers(0, S, size=40).tolist()))
    worst_o = worst_l = 0.0
    for i in rows:
        lo = max(NS, i - W + 1)
        keys = list(range(min(NS, i + 1))) + list(range(lo, i + 1))
        L = len(keys)
        idx = torch.tensor(keys, device="cuda")
        kc = k[0, 0].index_select(0, idx).cpu()
        vc = v[0, 0].index_select(0, idx).cpu()
        qc = torch.zeros((L, D), dtype=q.dtype)
        qc[L - 1] = q[0, 0, i].cpu()
        # compact positions: sinks 0..ns-1, then the window ending at L - 1
        ns = min(NS, i + 1)
        O, Lse = ORACLE.attention_fwd(fa_inputs.to_f64(qc.reshape(1, 1, L, D)),
                                      fa_inputs.to_f64(kc.reshape(1, 1, L, D)),
                                      fa_inputs.to_f64(vc.reshape(1, 1, L, D)), causal=True,
                                      scale=scale, window=(L - ns) if i >= NS else 0,
                                      n_sink=ns if i >= NS else 0, rows=[L - 1])
        og = o[0, 0, i].float().cpu().double().numpy()
        lg = float(lse[0, 0, i].cpu())
        worst_o = max(worst_o, float(np.abs(og - O[0, 0, 0]).max()))
        worst_l = max(worst_l, abs(lg - float(Lse[0, 0, 0])) / max(1.0, abs(float(Lse[0, 0, 0]))))
    _say(f"  long sequence S={S}: max|dO|={worst_o:.3e}  max rel dLSE={worst_l:.3e}")
    assert worst_o <= TOL_O["bf16"] and worst_l <= TOL_LSE_REL
    assert torch.isfinite(lse).all()
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_hip_graph_capture_and_replay():
    """Every call only enqueues kernels on the current stream (no allocation
    with caller-provided buffers, no memset, no host synchronisation), so the
    forward, the key-split forward with its merge, and the backward can be
    captured into one HIP graph. Each replay, with eager work and
    synchronisations in between, must equal the eager results bitwise."""
    B, H, S, D = 2, 4, 700, 128
    q, k, v = (t.cuda() for t in fa_inputs.make_qkv(B, H, S, D, "bf16", seed=21))
    dout = fa_inputs.make_qkv(B, H, S, D, "bf16", seed=22)[0].cuda()
    kw = dict(causal=True, window=300, n_sink=4)
    o_ref, l_ref = fa.flash_attn_fwd(q, k, v, **kw)
    os_ref, ls_ref = fa.flash_attn_fwd_split(q, k, v, n_split=3, **kw)
    g_ref = fa.flash_attn_bwd(q, k, v, o_ref, l_ref, dout, **kw)
    torch.cuda.synchronize()

    o, os_, dq, dk, dv = (torch.empty_like(q) for _ in range(5))
    l, ls_ = (torch.empty((B, H, S), dtype=torch.float32, device="cuda") for _ in range(2))
    ws_split = torch.empty(fa.flash_attn_split_workspace_bytes(B, H, S, D, 3), dtype=torch.uint8,
                           device="cuda")
    ws_bwd = torch.empty(fa.flash_attn_bwd_workspace_bytes(B, H, S), dtype=torch.uint8,
                         device="cuda")

    def calls():
        fa.flash_attn_fwd(q, k, v, out=o, lse=l, **kw)
        fa.flash_attn_fwd_split(q, k, v, n_split=3, workspace=ws_split, out=os_, lse=ls_, **kw)
        fa.flash_attn_bwd(q, k, v, o, l, dout, workspace=ws_bwd, dq=dq, dk=dk, dv=dv, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    outs = (o, l, os_, ls_, dq, dk, dv)
    refs = (o_ref, l_ref, os_ref, ls_ref) + tuple(g_ref)
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("o", "lse", "o split", "lse split", "dq", "dk", "dv"), outs, refs):
            assert torch.equal(t, r), (rep, name)
    _say("  graph: 4 replays bitwise equal to the eager calls")


def test_random_configurations():
    """A seeded sweep over combinations the targeted tests cover one at a time:
    batch, query and K/V heads, ragged S, D, dtype, mask (none, causal, window,
    sinks), ALiBi, the sign and size of the scale, and plain vs key-split
    forward. Each is checked against the oracle on every row."""
    rng = np.random.default_rng(2024)
    for n in range(36):
        dtype = ["bf16", "f16", "f32"][n % 3]
        D = int(rng.choice([16, 32, 64, 128])) if dtype == "f32" else int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 3]))
        B = int(rng.integers(1, 3))
        S = int(rng.integers(1, 520))
        causal = bool(rng.integers(0, 4) > 0)
        window = int(rng.integers(1, 300)) if causal and rng.random() < 0.5 else 0
        n_sink = int(rng.integers(0, 9)) if window else 0
        # within 1.5x of the usual 1/sqrt(D): sharper rows put |O| near the largest
        # |v|, where rounding O to bf16 alone approaches the bf16 bar (the sharp
        # softmax tests cover that regime with their own inputs)
        scale = float(rng.choice([1.0, -1.0]) * rng.uniform(0.1, 1.5) / math.sqrt(D))
        slopes = rng.uniform(-0.5, 1.5, size=H).astype(np.float32) if rng.random() < 0.4 else None
        split = int(rng.integers(2, 5)) if dtype != "f32" and rng.random() < 0.3 else 0
        q, _, _ = fa_inputs.make_qkv(B, H, S, D, dtype, seed=1000 + n)
        k, v = _kv(B, Hkv, S, D, dtype, seed=2000 + n)
        sd = None if slopes is None else torch.from_numpy(slopes).cuda()
        kw = dict(causal=causal, window=window, n_sink=n_sink, scale=scale, alibi_slopes=sd)
        label = (f"#{n} {dtype} B{B} H{H}/{Hkv} S{S} D{D} c{int(causal)} w{window} s{n_sink} "
                 f"scale {scale:+.3f} alibi {slopes is not None} split {split}")
        if split:
            o, lse = fa.flash_attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), n_split=split, **kw)
            torch.cuda.synchronize()
        else:
            o, lse = gpu_fwd(q, k, v, **kw)
        # fp32 rounding of the scores grows with their size: scale the fp32 bar
        # by |scale| sqrt(D), which is 1 at the usual 1/sqrt(D)
        tol = TOL_O["f32"] * max(1.0, abs(scale) * math.sqrt(D)) if dtype == "f32" else None
        compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                n_sink=n_sink, label=label, tol_o=tol,
                alibi=None if slopes is None else slopes.astype(np.float64))


def test_random_configurations_sharp_rows():
    """The sweep above with scales of 1.5 to 8 times 1/sqrt(D) (bf16, f16):
    rows concentrate on a few keys, the running max moves by large steps and
    |O| approaches the largest |v|. The bar adds to the dtype's bar the
    rounding of O itself to the output type, half an ulp: at most 2^-8 |O|
    (bf16) or 2^-11 |O| (f16), element by element. LSE keeps its bar."""
    rng = np.random.default_rng(77)
    rel = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
    for n in range(16):
        dtype = ["bf16", "f16"][n % 2]
        D = int(rng.choice([64, 128]))
        H, B = int(rng.choice([1, 2])), 1
        S = int(rng.integers(1, 700))
        causal = bool(rng.integers(0, 3) > 0)
        window = int(rng.integers(1, 300)) if causal and rng.random() < 0.4 else 0
        n_sink = int(rng.integers(0, 5)) if window else 0
        scale = float(rng.choice([1.0, -1.0]) * rng.uniform(1.5, 8.0) / math.sqrt(D))
        q, k, v = fa_inputs.make_qkv(B, H, S, D, dtype, seed=5000 + n)
        label = (f"sharp #{n} {dtype} H{H} S{S} D{D} c{int(causal)} w{window} s{n_sink} "
                 f"scale {scale:+.3f}")
        o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink, scale=scale)
        worst_excess, worst_l = -1.0, 0.0
        for h in range(H):
            O, L = ORACLE.attention_fwd(fa_inputs.to_f64(q[:, h:h + 1]),
                                        fa_inputs.to_f64(k[:, h:h + 1]),
                                        fa_inputs.to_f64(v[:, h:h + 1]), causal=causal,
                                        scale=scale, window=window, n_sink=n_sink)
            og = o[0, h].float().cpu().double().numpy()
            lg = lse[0, h].cpu().double().numpy()
            bar = TOL_O[dtype] + rel[dtype] * np.abs(O[0, 0])
            worst_excess = max(worst_excess, float((np.abs(og - O[0, 0]) - bar).max()))
            worst_l = max(worst_l, float((np.abs(lg - L[0, 0]) /
                                          np.maximum(1.0, np.abs(L[0, 0]))).max()))
        _say(f"  {label}: max(|dO| - bar)={worst_excess:.3e}  max rel dLSE={worst_l:.3e}")
        assert worst_excess <= 0.0, label
        assert worst_l <= TOL_LSE_REL, label


# --------------------------------------------------------------------------- #
# Ragged lengths, head dims, dtypes, masks
# --------------------------------------------------------------------------- #

MASKS = [(False, 0, 0), (True, 0, 0), (True, 100, 4), (True, 33, 0), (True, 64, 70)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_ragged_lengths(dtype, D):
    for S in (1, 7, 63, 65, 127, 129, 200, 1000):
        q, k, v = fa_inputs.make_qkv(1, 2, S, D, dtype, seed=S + D)
        for causal, window, n_sink in MASKS:
            scale = 1.0 / math.sqrt(D)
            o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink, scale=scale)
            compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                    n_sink=n_sink, label=f"{dtype} D{D} S{S} c{int(causal)} w{window} s{n_sink}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_multi_batch_head_layout(dtype):
    """B and H index distinct heads: B=3, H=5, ragged S."""
    q, k, v = fa_inputs.make_qkv(3, 5, 300, 64, dtype, seed=7)
    for causal in (False, True):
        o, lse = gpu_fwd(q, k, v, causal=causal, scale=0.125)
        compare(o, lse, q, k, v, dtype, causal=causal, scale=0.125, label=f"{dtype} B3H5 c{causal}")


def test_work_group_order_uneven_groups():
    """B*H = 40: eight XCD runs of five heads each, which the causal order splits
    into groups of four and one. Every (query block, head) must still be
    computed once: the small-grid schedule, the 4-wave kernel (ALiBi) and the
    backward, all on every row against the oracle."""
    B, H, S, D = 5, 8, 300, 128
    q, k, v = fa_inputs.make_qkv(B, H, S, D, "bf16", seed=40)
    sl = ORACLE.alibi_slopes(H).astype(np.float32)
    for slopes in (None, sl):
        sd = None if slopes is None else torch.from_numpy(slopes).cuda()
        o, lse = gpu_fwd(q, k, v, causal=True, scale=0.088, alibi_slopes=sd)
        compare(o, lse, q, k, v, "bf16", causal=True, scale=0.088,
                alibi=None if slopes is None else slopes.astype(np.float64),
                label=f"B5H8 causal alibi={slopes is not None}")
    _bwd_case(B, H, H, S, D, "bf16", True, 0, 0, 0.088, seed=41, label="B5H8 backward")


# --------------------------------------------------------------------------- #
# Stress inputs and degenerate cases
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_sharp_softmax_and_key_offset(dtype):
    """Q x 8 gives nearly one-hot rows (large rescales); a common key offset
    shifts every score of a row by the same amount (O unchanged)."""
    q, k, v = fa_inputs.make_qkv(1, 2, 520, 128, dtype, seed=3)
    tdt = q.dtype
    q8 = (q.float() * 8).to(tdt)
    o, lse = gpu_fwd(q8, k, v, causal=True, scale=1 / math.sqrt(128))
    # In fp32 the scores themselves carry a rounding error of order
    # eps32 * |s| * sqrt(D); scaling Q by 8 scales that error, and so the
    # error of every softmax weight, by 8, so the fp32 bar scales with it.
    # (For f16/bf16 the bar is set by rounding P and O to 8-/11-bit
    # mantissas, which does not grow with the score magnitude.)
    tol = TOL_O[dtype] * 8 if dtype == "f32" else None
    compare(o, lse, q8, k, v, dtype, causal=True, scale=1 / math.sqrt(128), label=f"{dtype} Qx8",
            tol_o=tol)
    off = torch.from_numpy(np.random.default_rng(0).standard_normal(128).astype(np.float32) * 4)
    k2 = (k.float() + off).to(tdt)
    o2, lse2 = gpu_fwd(q, k2, v, causal=True, scale=1 / math.sqrt(128))
    compare(o2, lse2, q, k2, v, dtype, causal=True, scale=1 / math.sqrt(128),
            label=f"{dtype} key offset")


def _spiked_inputs(B, H, S, D, dtype, seed, pattern):
    """Q, K, V whose scores jump far above everything before them at chosen
    keys: Q gains a common direction u (|u| = 1, q.u about 4), and key j gains
    g_j u, which lifts its score against every query by about 4 g_j / sqrt(D)
    (natural-log units at scale 1/sqrt(D)). "spikes": keys 300, 700 and 1000
    jump by 20, 40 and 60; "ramp": every key j rises by 20 per 64-key block
    over the previous block."""
    q, k, v = fa_inputs.make_qkv(B, H, S, D, "f32", seed=seed)
    u = torch.from_numpy(np.random.default_rng(seed + 100).standard_normal(D).astype(np.float32))
    u = u / u.norm()
    q = q + 4.0 * u
    g = torch.zeros(S)
    if pattern == "spikes":
        for j, lift in ((300, 20.0), (700, 40.0), (1000, 60.0)):
            if j < S:
                g[j] = lift * math.sqrt(D) / 4.0
    else:
        g = torch.div(torch.arange(S), 64, rounding_mode="floor").float() * 20.0 * math.sqrt(D) / 4.0
    k = k + g[None, None, :, None] * u
    tdt = fa_inputs.DTYPES[dtype]
    return q.to(tdt), k.to(tdt), v.to(tdt)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pattern", ["spikes", "ramp"])
def test_score_jumps_in_visible_blocks(dtype, D, pattern):
    """Scores that jump far above the running max inside fully visible blocks,
    deep in the sequence: the kernel's lazy rescale keeps a stale reference
    max until a block's max exceeds it by more than 2^8 (base 2), so each
    jump must move the reference and rescale O and l at once (a weight formed
    against the old reference would overflow fp32, or f16). Single jumps of
    20, 40 and 60 (natural-log units) and a ramp that rises by 20 every block;
    causal, with a window and sinks, with a key split, with ALiBi, and
    without a mask."""
    S = 1100 if pattern == "spikes" else 700
    q, k, v = _spiked_inputs(1, 2, S, D, dtype, seed=21, pattern=pattern)
    scale = 1.0 / math.sqrt(D)
    o, lse = gpu_fwd(q, k, v, causal=True, scale=scale)
    compare(o, lse, q, k, v, dtype, causal=True, scale=scale, label=f"{dtype} D{D} {pattern}")
    o, lse = gpu_fwd(q, k, v, causal=True, window=500, n_sink=3, scale=scale)
    compare(o, lse, q, k, v, dtype, causal=True, window=500, n_sink=3, scale=scale,
            label=f"{dtype} D{D} {pattern} window")
    o, lse = fa.flash_attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), n_split=3, causal=True,
                                     scale=scale)
    torch.cuda.synchronize()
    compare(o, lse, q, k, v, dtype, causal=True, scale=scale, label=f"{dtype} D{D} {pattern} split")
    slopes = np.array([0.01, 0.002], dtype=np.float32)
    o, lse = gpu_fwd(q, k, v, causal=True, scale=scale, alibi_slopes=torch.from_numpy(slopes).cuda())
    compare(o, lse, q, k, v, dtype, causal=True, scale=scale, alibi=slopes.astype(np.float64),
            label=f"{dtype} D{D} {pattern} alibi")
    o, lse = gpu_fwd(q, k, v, causal=False, scale=scale)
    compare(o, lse, q, k, v, dtype, causal=False, scale=scale, label=f"{dtype} D{D} {pattern} full")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_zero_and_negative(dtype):
    """scale = 0: every visible key weighs the same (O = mean of visible V,
    LSE = ln count). A negative scale is a valid multiplier too."""
    q, k, v = fa_inputs.make_qkv(1, 2, 150, 64, dtype, seed=11)
    for causal, window, n_sink in MASKS:
        for scale in (0.0, -0.2):
            o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink, scale=scale)
            compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                    n_sink=n_sink, label=f"{dtype} scale={scale} c{causal} w{window}")


def test_window_one_and_wide_window():
    """window = 1 without sinks: each row sees only itself (O = V exactly);
    a window wider than S is plain causal."""
    q, k, v = fa_inputs.make_qkv(1, 3, 257, 128, "bf16", seed=5)
    o, lse = gpu_fwd(q, k, v, causal=True, window=1, scale=0.1)
    assert torch.equal(o.cpu(), v)
    o1, l1 = gpu_fwd(q, k, v, causal=True, window=0, scale=0.1)
    o2, l2 = gpu_fwd(q, k, v, causal=True, window=5000, n_sink=3, scale=0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_self_attention_aliasing_and_side_stream():
    """q, k and v may be one tensor; the launch follows torch's current stream."""
    x, _, _ = fa_inputs.make_qkv(2, 4, 333, 64, "f16", seed=9)
    xd = x.cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.flash_attn_fwd(xd, xd, xd, causal=True, scale=0.125)
    s.synchronize()
    compare(o, lse, x, x, x, "f16", causal=True, scale=0.125, label="aliased q=k=v, side stream")


def test_preallocated_outputs_fully_written():
    q, k, v = fa_inputs.make_qkv(1, 2, 77, 32, "bf16", seed=2)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((1, 2, 77), float("nan"), device="cuda")
    fa.flash_attn_fwd(qd, kd, vd, causal=True, out=out, lse=lse, scale=0.3)
    torch.cuda.synchronize()
    compare(out, lse, q, k, v, "bf16", causal=True, scale=0.3, label="preallocated outputs")


def test_deterministic_bitwise():
    q, k, v = fa_inputs.make_qkv(2, 4, 1000, 128, "bf16", seed=4)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    ref = fa.flash_attn_fwd(qd, kd, vd, causal=True, window=300, n_sink=4)
    for _ in range(10):
        o, l = fa.flash_attn_fwd(qd, kd, vd, causal=True, window=300, n_sink=4)
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])


def test_grid_order_reversal_bitwise():
    """No work-group depends on another, so dispatching the work-groups in the
    opposite order (FLASH_ATTN_REVERSE_ORDER=1, read per call) must give
    bitwise the same O and LSE: causal, window with sinks, no mask, grouped
    heads with ALiBi, a key split, the 8-wave kernel and the generic f32
    kernel."""
    cases = [
        dict(shape=(2, 4, 1000, 128), dtype="bf16", kw=dict(causal=True)),
        dict(shape=(2, 4, 1000, 128), dtype="bf16", kw=dict(causal=True, window=300, n_sink=4)),
        dict(shape=(1, 8, 777, 64), dtype="f16", kw=dict(causal=False)),
        dict(shape=(1, 8, 900, 128), dtype="bf16", kv=2, alibi=True, kw=dict(causal=True)),
        dict(shape=(1, 4, 1500, 128), dtype="bf16", split=3, kw=dict(causal=True)),
        dict(shape=(1, 64, 16384, 128), dtype="bf16", kw=dict(causal=True)),
        dict(shape=(1, 2, 300, 32), dtype="f32", kw=dict(causal=True)),
    ]
    for c in cases:
        B, H, S, D = c["shape"]
        q, k, v = fa_inputs.make_qkv(B, H, S, D, c["dtype"], seed=8, H_kv=c.get("kv", 0))
        qd, kd, vd = (t.cuda() for t in (q, k, v))
        sl = torch.from_numpy(ORACLE.alibi_slopes(H).astype(np.float32)).cuda() \
            if c.get("alibi") else None

        def run():
            if c.get("split"):
                return fa.flash_attn_fwd_split(qd, kd, vd, n_split=c["split"], **c["kw"])
            return fa.flash_attn_fwd(qd, kd, vd, alibi_slopes=sl, **c["kw"])

        ref = run()
        os.environ["FLASH_ATTN_REVERSE_ORDER"] = "1"
        try:
            rev = run()
        finally:
            del os.environ["FLASH_ATTN_REVERSE_ORDER"]
        torch.cuda.synchronize()
        _say(f"  reversed dispatch order {c['shape']} {c['dtype']} {c['kw']}: "
             f"equal={torch.equal(ref[0], rev[0]) and torch.equal(ref[1], rev[1])}")
        assert torch.equal(ref[0], rev[0]) and torch.equal(ref[1], rev[1]), c


@pytest.mark.parametrize("parts, dtype, D", [("0", "bf16", 128), ("2", "bf16", 128),
                                             ("0", "f16", 64), ("2", "f16", 64), ("4", "f16", 64),
                                             ("4", "bf16", 64)])
def test_every_small_grid_schedule(parts, dtype, D):
    """Grids of fewer than 512 work-groups of 128 rows take the small-grid
    schedule by default (no ALiBi, no key split): two key parts, or four on
    64-row blocks at D = 64 when the grid covers at most half the CUs.
    FLASH_ATTN_PARTS=0|2|4, read per call, forces a schedule. Each against
    the oracle: the 4-wave kernel keeps its small-size coverage, and the
    key-part kernels meet parts with no visible key (one key block, a narrow
    window), uneven block counts and ragged tails. Sink counts 32 and 33
    straddle the 4-wave kernel's half-width sink step (taken when every sink
    lies in the first 32 keys of the sink block)."""
    os.environ["FLASH_ATTN_PARTS"] = parts
    try:
        for S in (1, 64, 65, 129, 700, 1000):
            q, k, v = fa_inputs.make_qkv(1, 2, S, D, dtype, seed=S + 11 * D)
            for causal, window, n_sink in MASKS + [(True, 200, 32), (True, 200, 33)]:
                scale = 1.0 / math.sqrt(D)
                o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink, scale=scale)
                compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                        n_sink=n_sink,
                        label=f"parts={parts} {dtype} D{D} S{S} c{int(causal)} w{window} s{n_sink}")
    finally:
        del os.environ["FLASH_ATTN_PARTS"]


# --------------------------------------------------------------------------- #
# Block skipping: the instrumentation counter against a count from the mask
# --------------------------------------------------------------------------- #

def _pairs_with_visible_keys(S, bq, bk, causal, window, n_sink):
    total = 0
    for q0 in range(0, S, bq):
        rows = np.arange(q0, min(S, q0 + bq))
        keep = ORACLE.visible(rows, S, causal, window, n_sink)
        for k0 in range(0, S, bk):
            total += bool(keep[:, k0:k0 + bk].any())
    return total


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S,causal,window,n_sink", [
    (64, True, 0, 0), (4096, True, 0, 0), (4096, False, 0, 0), (1000, True, 0, 0),
    (8192, True, 1024, 4), (3000, True, 200, 70), (3000, True, 200, 0)])
def test_block_pairs_visited(S, causal, window, n_sink, D):
    bq, bk = fa.flash_attn_tile_shape(1, 1, S, D, fa.FA_BF16, window=window)
    q, k, v = fa_inputs.make_qkv(1, 1, S, D, "bf16", seed=1)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    fa.flash_attn_fwd_counted(qd, kd, vd, cnt, causal=causal, window=window, n_sink=n_sink)
    torch.cuda.synchronize()
    want = _pairs_with_visible_keys(S, bq, bk, causal, window, n_sink)
    nq, nk = -(-S // bq), -(-S // bk)
    _say(f"  S={S} causal={causal} w={window} sinks={n_sink}: visited {int(cnt.item())} "
         f"of {nq * nk} tile pairs (mask-derived {want})")
    assert int(cnt.item()) == want


def test_invalid_arguments_raise_before_launch():
    q, k, v = (t.cuda() for t in fa_inputs.make_qkv(1, 1, 16, 64, "bf16"))
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, k, v, causal=False, window=4)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, k, v, scale=float("nan"))
    with pytest.raises(NotImplementedError):
        x = torch.zeros(1, 1, 16, 48, dtype=torch.bfloat16, device="cuda")
        fa.flash_attn_fwd(x, x, x)


def test_tiled_block_guide_example_fp32():
    """The NumPy tiled-block guide's validation case (non-causal, N=512,
    d=64, seed 42, fp32) through the fp32 path, within its asserted 1e-4."""
    rng = np.random.default_rng(42)
    arrs = [rng.normal(size=(512, 64)).astype(np.float32) for _ in range(3)]
    q, k, v = (torch.from_numpy(a).reshape(1, 1, 512, 64) for a in arrs)
    o, lse = gpu_fwd(q, k, v, causal=False, scale=0.125)
    worst, _ = compare(o, lse, q, k, v, "f32", causal=False, scale=0.125, label="guide fp32")
    assert worst < 1e-4


# --------------------------------------------------------------------------- #
# Grouped key/value heads (MQA / GQA) and the ALiBi bias
# --------------------------------------------------------------------------- #

def _kv(B, Hkv, S, D, dtype, seed):
    _, k, v = fa_inputs.make_qkv(B, Hkv, S, D, dtype, seed=seed)
    return k, v


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_grouped_kv_heads(dtype, D):
    """Query head h reads key/value head h // (H // H_kv): H = 8 with H_kv = 1
    (multi-query), 2, 4 and 8, at B = 2 so that B*H is a multiple of 8."""
    for S in (200, 1000):
        q, _, _ = fa_inputs.make_qkv(2, 8, S, D, dtype, seed=S + 3)
        for Hkv in (1, 2, 4, 8):
            k, v = _kv(2, Hkv, S, D, dtype, seed=S + Hkv)
            for causal, window, n_sink in MASKS[:3]:
                scale = 1.0 / math.sqrt(D)
                o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink,
                                 scale=scale)
                heads = [(b, h) for b in range(2) for h in range(8)] if S <= 200 else \
                    [(0, 0), (0, 7), (1, 3), (1, 6)]
                compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                        n_sink=n_sink, heads=heads,
                        label=f"{dtype} D{D} S{S} H8/Hkv{Hkv} c{int(causal)} w{window}")


def test_grouped_heads_equal_repeated_heads_bitwise():
    """A grouped call and an ordinary call on explicitly repeated K/V heads run
    the same arithmetic, so they agree bit for bit."""
    q, _, _ = fa_inputs.make_qkv(2, 8, 333, 128, "bf16", seed=5)
    k, v = _kv(2, 2, 333, 128, "bf16", seed=6)
    o1, l1 = gpu_fwd(q, k, v, causal=True, scale=0.088)
    o2, l2 = gpu_fwd(q, k.repeat_interleave(4, dim=1).contiguous(),
                     v.repeat_interleave(4, dim=1).contiguous(), causal=True, scale=0.088)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_alibi(dtype, D):
    """ALiBi slopes of the Lesson 91 rule (and a steep / a zero slope) under
    every mask, alone and with grouped heads."""
    H = 4
    slopes = np.array(list(ORACLE.alibi_slopes(H)), dtype=np.float32)
    steep = np.array([1.5, 0.0, 0.3, 2.0 ** -8], dtype=np.float32)
    for S in (129, 700):
        q, _, _ = fa_inputs.make_qkv(2, H, S, D, dtype, seed=S + 11)
        for Hkv in (H, 2):
            k, v = _kv(2, Hkv, S, D, dtype, seed=S + 12 + Hkv)
            for sl in (slopes, steep):
                sd = torch.from_numpy(sl).cuda()
                for causal, window, n_sink in MASKS[:3]:
                    scale = 1.0 / math.sqrt(D)
                    o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink,
                                     scale=scale, alibi_slopes=sd)
                    compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                            n_sink=n_sink, alibi=sl.astype(np.float64),
                            label=f"{dtype} D{D} S{S} alibi Hkv{Hkv} c{int(causal)} w{window}")


def test_alibi_negative_scale_and_zero_scale():
    """The bias is added after the (signed) scale; with scale 0 only the bias
    remains (the oracle's geometric closed form)."""
    H = 4
    sl = np.array(list(ORACLE.alibi_slopes(H)), dtype=np.float32)
    sd = torch.from_numpy(sl).cuda()
    q, k, v = fa_inputs.make_qkv(1, H, 300, 64, "bf16", seed=21)
    for scale in (-0.2, 0.0):
        for causal in (False, True):
            o, lse = gpu_fwd(q, k, v, causal=causal, scale=scale, alibi_slopes=sd)
            compare(o, lse, q, k, v, "bf16", causal=causal, scale=scale,
                    alibi=sl.astype(np.float64), label=f"alibi scale {scale} c{int(causal)}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_alibi_slope_range_causal(dtype):
    """Under the causal mask the fast kernel adds the bias in a linear form for
    moderate slopes and per score for steep ones (|slope log2 e| > 16): slopes
    on both sides of that switch, negative and very large ones, with the
    reversed block walk, a ragged tail and a window."""
    H = 8
    sl = np.array([0.5, -0.3, 11.0, 11.2, 40.0, 1e3, 1e30, -2.0], dtype=np.float32)
    sd = torch.from_numpy(sl).cuda()
    for S, window, n_sink in ((333, 0, 0), (700, 150, 3)):
        q, k, v = fa_inputs.make_qkv(1, H, S, 128, dtype, seed=S + 40)
        scale = 1.0 / math.sqrt(128)
        o, lse = gpu_fwd(q, k, v, causal=True, window=window, n_sink=n_sink, scale=scale,
                         alibi_slopes=sd)
        compare(o, lse, q, k, v, dtype, causal=True, scale=scale, window=window, n_sink=n_sink,
                alibi=sl.astype(np.float64), label=f"{dtype} S{S} w{window} alibi slope range")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_head_dim_64_full_grid(dtype):
    """D = 64 on a grid of 512 work-groups of 128 rows (B2 H16 S2048), which
    takes the 4-wave kernel built for three waves per SIMD rather than the
    small-grid schedule; no mask, causal, and a window with sinks, each checked
    on every row of three heads."""
    assert fa.flash_attn_fwd_kernel(2, 16, 2048, 64, fa.FA_BF16).startswith(
        "fa_fwd_fast_kernel<bf16,D=64,waves=4>")
    q, k, v = fa_inputs.make_qkv(2, 16, 2048, 64, dtype, seed=64)
    heads = [(0, 0), (1, 15), (1, 6)]
    for causal, window, n_sink in ((False, 0, 0), (True, 0, 0), (True, 300, 3)):
        o, lse = gpu_fwd(q, k, v, causal=causal, window=window, n_sink=n_sink, scale=0.125)
        compare(o, lse, q, k, v, dtype, causal=causal, scale=0.125, window=window,
                n_sink=n_sink, heads=heads, label=f"{dtype} D64 B2H16 S2048 c{int(causal)} w{window}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_head_dim_128_eight_wave_plan(dtype):
    """D = 128 without a window from S = 2048 on a grid of 512 work-groups of
    256 rows (B4 H16 S2048): the plan takes the 8-wave kernel by itself; no
    mask, causal, causal with grouped heads, and a ragged length (S 2100, whose
    last block holds 52 rows), each checked on every row of three heads. A
    window on the same grid keeps 4 waves."""
    for dt in (fa.FA_BF16, fa.FA_F16):
        assert "waves=8" in fa.flash_attn_fwd_kernel(4, 16, 2048, 128, dt)
        assert "waves=8" in fa.flash_attn_fwd_kernel(4, 16, 2100, 128, dt)
        assert "waves=4" in fa.flash_attn_fwd_kernel(4, 16, 2048, 128, dt, window=512)
    heads = [(0, 0), (3, 15), (2, 9)]
    for S, Hkv, causal in ((2048, 16, False), (2048, 16, True), (2048, 4, True), (2100, 16, True)):
        q, _, _ = fa_inputs.make_qkv(4, 16, S, 128, dtype, seed=S + Hkv)
        k, v = _kv(4, Hkv, S, 128, dtype, seed=S + Hkv + 1)
        scale = 1.0 / math.sqrt(128)
        o, lse = gpu_fwd(q, k, v, causal=causal, scale=scale)
        compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, heads=heads,
                label=f"{dtype} D128 B4H16 Hkv{Hkv} S{S} c{int(causal)} (8 waves by plan)")


def test_eight_wave_work_groups():
    """The 8-wave (256-row) work-groups that long sequences and D = 128 without
    a window use, forced on shorter ones: ALiBi under the causal mask (backward
    walk), a window with sinks, grouped heads and a ragged tail."""
    old = os.environ.get("FLASH_ATTN_WAVES")
    os.environ["FLASH_ATTN_WAVES"] = "8"
    try:
        H = 4
        sl = np.array(list(ORACLE.alibi_slopes(H)), dtype=np.float32)
        sd = torch.from_numpy(sl).cuda()
        for dtype, D, S, Hkv, window, n_sink, al in (("bf16", 128, 611, 4, 0, 0, True),
                                                    ("f16", 128, 700, 2, 200, 4, False),
                                                    ("bf16", 64, 530, 1, 0, 0, False),
                                                    ("f16", 64, 333, 2, 90, 3, True)):
            q, _, _ = fa_inputs.make_qkv(1, H, S, D, dtype, seed=S + 3)
            k, v = _kv(1, Hkv, S, D, dtype, seed=S + 4)
            scale = 1.0 / math.sqrt(D)
            o, lse = gpu_fwd(q, k, v, causal=True, window=window, n_sink=n_sink, scale=scale,
                             alibi_slopes=sd if al else None)
            compare(o, lse, q, k, v, dtype, causal=True, scale=scale, window=window,
                    n_sink=n_sink, alibi=sl.astype(np.float64) if al else None,
                    label=f"8 waves {dtype} D{D} S{S} Hkv{Hkv} w{window} alibi {al}")
    finally:
        if old is None:
            del os.environ["FLASH_ATTN_WAVES"]
        else:
            os.environ["FLASH_ATTN_WAVES"] = old


def test_alibi_rejects_bad_slopes_tensor():
    q, k, v = (t.cuda() for t in fa_inputs.make_qkv(1, 4, 64, 64, "bf16", seed=1))
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, k, v, alibi_slopes=torch.zeros(3, device="cuda"))
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(q, k, v, alibi_slopes=torch.zeros(4, dtype=torch.float64,
                                                             device="cuda"))


# --------------------------------------------------------------------------- #
# Key-split partials and the merge
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_split_keys(dtype, D):
    """flash_attn_fwd_split against the oracle for several split counts (more
    splits than key blocks included), every mask, ragged S, grouped heads and
    ALiBi."""
    for S in (100, 700, 1029):
        q, _, _ = fa_inputs.make_qkv(2, 4, S, D, dtype, seed=S + 31)
        k, v = _kv(2, 2, S, D, dtype, seed=S + 32)
        for n_split in (1, 2, 3, 7):
            for causal, window, n_sink in MASKS[:3]:
                scale = 1.0 / math.sqrt(D)
                qd, kd, vd = (t.cuda() for t in (q, k, v))
                o, lse = fa.flash_attn_fwd_split(qd, kd, vd, n_split=n_split, causal=causal,
                                                 window=window, n_sink=n_sink, scale=scale)
                torch.cuda.synchronize()
                compare(o, lse, q, k, v, dtype, causal=causal, scale=scale, window=window,
                        n_sink=n_sink, heads=[(0, 0), (1, 3)],
                        label=f"{dtype} D{D} S{S} split{n_split} c{int(causal)} w{window}")
    # with ALiBi
    q, k, v = fa_inputs.make_qkv(1, 4, 500, D, dtype, seed=77)
    sl = np.array(list(ORACLE.alibi_slopes(4)), dtype=np.float32)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.flash_attn_fwd_split(qd, kd, vd, n_split=3, causal=True, scale=0.1,
                                     alibi_slopes=torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    compare(o, lse, q, k, v, dtype, causal=True, scale=0.1, alibi=sl.astype(np.float64),
            label=f"{dtype} D{D} split3 alibi")


def test_split_workspace_reuse_and_block_count():
    """One caller-owned workspace serves consecutive calls of different sizes;
    the block counter of split work-groups adds up to the unsplit count."""
    q, k, v = (t.cuda() for t in fa_inputs.make_qkv(2, 8, 1024, 64, "f16", seed=5))
    need = fa.flash_attn_split_workspace_bytes(2, 8, 1024, 64, 4)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # garbage contents
    o1, l1 = fa.flash_attn_fwd_split(q, k, v, n_split=4, causal=False, scale=0.125, workspace=ws)
    o2, l2 = fa.flash_attn_fwd(q, k, v, causal=False, scale=0.125)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2 * TOL_O["f16"]
    assert (l1 - l2).abs().max().item() <= 1e-4
    qs, ks, vs = (t[:, :, :300].contiguous() for t in (q, k, v))
    o3, l3 = fa.flash_attn_fwd_split(qs, ks, vs, n_split=2, causal=True, scale=0.125, workspace=ws)
    torch.cuda.synchronize()
    compare(o3, l3, qs.cpu(), ks.cpu(), vs.cpu(), "f16", causal=True, scale=0.125,
            heads=[(0, 0), (1, 7)], label="split reuse smaller")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_merge_of_oracle_partials(dtype, D):
    """The merge kernel on partials the oracle computed (CPU, fp64 rounded to
    fp32) against the oracle's own merge: independent of the split kernel."""
    S, H = 90, 3
    q, k, v = fa_inputs.make_qkv(1, H, S, D, "f32", seed=D + 1)
    q64, k64, v64 = (fa_inputs.to_f64(t) for t in (q, k, v))
    cuts = [0, 13, 13, 50, 90]
    parts = [ORACLE.attention_fwd(q64, k64, v64, causal=True, scale=0.2, key_range=(a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    Op = np.stack([p_[0] for p_ in parts]).astype(np.float32)     # [n, 1, H, S, D]
    Lp = np.stack([p_[1] for p_ in parts]).astype(np.float32)     # [n, 1, H, S]
    Om, Lm = ORACLE.merge_partials(Op.astype(np.float64), Lp.astype(np.float64))
    o, lse = fa.flash_attn_merge(torch.from_numpy(Op).cuda(), torch.from_numpy(Lp).cuda(),
                                 dtype=fa_inputs.DTYPES[dtype])
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    # rounding: fp32 partials are exact inputs; fp32 arithmetic, then one
    # rounding to the output type
    tol = {"f32": 1e-5, "f16": 2e-3, "bf16": 8e-3}[dtype]
    assert np.abs(og - Om).max() <= tol
    assert np.abs(lg - Lm).max() <= 1e-5
    # every row of the range [13, 13) part is -inf; row 0 sees only part 0
    assert np.isinf(Lp[1]).all()


def test_merge_all_parts_empty():
    Op = torch.zeros(2, 5, 64, device="cuda")
    Lp = torch.full((2, 5), float("-inf"), device="cuda")
    Lp[1, 3] = 0.5
    Op[1, 3] = 2.0
    o, lse = fa.flash_attn_merge(Op, Lp)
    torch.cuda.synchronize()
    assert torch.isinf(lse[[0, 1, 2, 4]]).all() and (o[[0, 1, 2, 4]] == 0).all()
    assert lse[3].item() == pytest.approx(0.5) and torch.allclose(o[3], torch.full((64,), 2.0,
                                                                                  device="cuda"))


# --------------------------------------------------------------------------- #
# Backward
# --------------------------------------------------------------------------- #

# Gradient bars, normwise: max |d - d_ref| <= TOL_G * max(1, max |d_ref|) per
# tensor. P and dS are rounded to the input type (8- or 11-bit significand,
# relative 2^-9 / 2^-12) before the products; with fp32 accumulation over at
# most S terms of mixed sign, the error stays a few of those units of the
# tensor's scale, and the bars leave a factor of ~4 over 2^-9 / 2^-12 * 10.
TOL_G = {"bf16": 2.5e-2, "f16": 4e-3}


def _grad_err(got, ref):
    ref = np.asarray(ref)
    return float(np.abs(got.float().cpu().double().numpy() - ref).max() /
                 max(1.0, float(np.abs(ref).max())))


@pytest.fixture(params=["1", "2"])
def dkv_kernel(request):
    """Runs a backward test with each dK/dV kernel (FLASH_ATTN_DKV=1: one
    wave per SIMD, K/V in registers; 2: two waves per SIMD, K/V in LDS),
    read per call."""
    os.environ["FLASH_ATTN_DKV"] = request.param
    try:
        yield request.param
    finally:
        del os.environ["FLASH_ATTN_DKV"]


def _bwd_case(B, H, Hkv, S, D, dtype, causal, window, n_sink, scale, seed, slopes=None,
              heads=None, label=""):
    q, _, _ = fa_inputs.make_qkv(B, H, S, D, dtype, seed=seed)
    k, v = _kv(B, Hkv, S, D, dtype, seed=seed + 1)
    dout, _, _ = fa_inputs.make_qkv(B, H, S, D, dtype, seed=seed + 2)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    sd = None if slopes is None else torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    o, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window=window, n_sink=n_sink,
                               scale=scale, alibi_slopes=sd)
    dq, dk, dv = fa.flash_attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, window=window,
                                   n_sink=n_sink, scale=scale, alibi_slopes=sd)
    torch.cuda.synchronize()
    rq, rk, rv = ORACLE.attention_bwd(fa_inputs.to_f64(q), fa_inputs.to_f64(k),
                                      fa_inputs.to_f64(v), fa_inputs.to_f64(dout), causal=causal,
                                      scale=scale, window=window, n_sink=n_sink,
                                      alibi_slopes=slopes)
    eq, ek, ev = _grad_err(dq, rq), _grad_err(dk, rk), _grad_err(dv, rv)
    _say(f"  {label}: dq {eq:.2e} dk {ek:.2e} dv {ev:.2e} (tol {TOL_G[dtype]:g})")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(t.float()).all(), (label, name)
    assert max(eq, ek, ev) <= TOL_G[dtype], (label, eq, ek, ev)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_backward(dtype, D, dkv_kernel):
    for S in (1, 63, 200, 333):
        for causal, window, n_sink in MASKS:
            _bwd_case(1, 2, 2, S, D, dtype, causal, window, n_sink, 1.0 / math.sqrt(D),
                      seed=S + D, label=f"{dtype} D{D} S{S} c{int(causal)} w{window} s{n_sink}")


def test_backward_random_configurations(dkv_kernel):
    """A seeded sweep of the backward over batch, grouped heads, ragged S, D,
    dtype, mask, ALiBi and the scale's sign, each against the oracle's
    gradients."""
    rng = np.random.default_rng(77)
    for n in range(14):
        dtype = ["bf16", "f16"][n % 2]
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2]))
        B = int(rng.integers(1, 3))
        S = int(rng.integers(1, 300))
        causal = bool(rng.integers(0, 4) > 0)
        window = int(rng.integers(1, 200)) if causal and rng.random() < 0.5 else 0
        n_sink = int(rng.integers(0, 6)) if window else 0
        scale = float(rng.choice([1.0, -1.0]) * rng.uniform(0.3, 1.5) / math.sqrt(D))
        slopes = rng.uniform(-0.3, 1.2, size=H) if rng.random() < 0.4 else None
        _bwd_case(B, H, Hkv, S, D, dtype, causal, window, n_sink, scale, seed=5000 + 10 * n,
                  slopes=slopes,
                  label=f"#{n} {dtype} B{B} H{H}/{Hkv} S{S} D{D} c{int(causal)} w{window} "
                        f"s{n_sink} scale {scale:+.3f} alibi {slopes is not None}")


def test_backward_sequence_longer_than_2_to_the_24(dkv_kernel):
    """The backward on one head of S = 2^24 + 77 keys (4.3 GB per tensor) with a
    64-key window, checked on sampled rows against the oracle run on compact
    copies: dQ of row i needs only keys [i - W + 1, i]; dK and dV of key j need
    only the queries [j, j + W - 1], whose windows lie within [j - W + 1,
    j + W - 1]. The mask depends on i - j alone, so the compact problems keep
    those rows' visible sets and scores."""
    S, D, W = (1 << 24) + 77, 128, 64
    scale = 1.0 / math.sqrt(D)
    _say("long backward: generating inputs on the device")
    q, k, v = fa_inputs.make_qkv_device(S, D, "bf16", seed=31, device="cuda")
    dout = fa_inputs.make_qkv_device(S, D, "bf16", seed=32, device="cuda")[0]
    torch.cuda.empty_cache()
    o, lse = fa.flash_attn_fwd(q, k, v, causal=True, window=W, scale=scale)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, lse, dout, causal=True, window=W, scale=scale)
    torch.cuda.synchronize()
    del o, lse

    def compact(a, b):
        idx = torch.arange(a, b, device="cuda")
        return [fa_inputs.to_f64(t[0, 0].index_select(0, idx).cpu().reshape(1, 1, b - a, D))
                for t in (q, k, v, dout)]

    rng = np.random.default_rng(9)
    picks = sorted(set([0, 1, 63, 64, 65, S // 2, S - 64, S - 2, S - 1, (1 << 24) - 1, 1 << 24])
                   | set(rng.integers(0, S, size=30).tolist()))
    err = {"dq": [0.0, 1.0], "dk": [0.0, 1.0], "dv": [0.0, 1.0]}
    for i in picks:                       # dQ of row i
        a = max(0, i - W + 1)
        rq, _, _ = ORACLE.attention_bwd(*compact(a, i + 1), causal=True, scale=scale, window=W)
        got = dq[0, 0, i].float().cpu().double().numpy()
        err["dq"][0] = max(err["dq"][0], float(np.abs(got - rq[0, 0, i - a]).max()))
        err["dq"][1] = max(err["dq"][1], float(np.abs(rq[0, 0, i - a]).max()))
    for j in picks:                       # dK, dV of key j
        a, b = max(0, j - W + 1), min(S, j + W)
        _, rk, rv = ORACLE.attention_bwd(*compact(a, b), causal=True, scale=scale, window=W)
        for name, t, r in (("dk", dk, rk), ("dv", dv, rv)):
            got = t[0, 0, j].float().cpu().double().numpy()
            err[name][0] = max(err[name][0], float(np.abs(got - r[0, 0, j - a]).max()))
            err[name][1] = max(err[name][1], float(np.abs(r[0, 0, j - a]).max()))
    rel = {n: e / m for n, (e, m) in err.items()}
    _say("  long backward S=%d: " % S + " ".join(f"{n} {x:.2e}" for n, x in rel.items()))
    assert max(rel.values()) <= TOL_G["bf16"], rel
    del q, k, v, dout, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_grouped_heads_alibi_scale(dtype, dkv_kernel):
    """Grouped K/V heads (dk, dv sum over the group), ALiBi, negative and zero
    scale."""
    _bwd_case(2, 4, 2, 257, 128, dtype, True, 0, 0, 0.088, seed=3, label="gqa")
    _bwd_case(1, 4, 1, 190, 64, dtype, False, 0, 0, 0.125, seed=4, label="mqa")
    _bwd_case(1, 4, 2, 230, 128, dtype, True, 0, 0, 0.088, seed=5,
              slopes=ORACLE.alibi_slopes(4), label="alibi")
    _bwd_case(1, 4, 2, 230, 64, dtype, True, 0, 0, 0.125, seed=9,
              slopes=ORACLE.alibi_slopes(4), label="alibi D64")
    _bwd_case(1, 2, 2, 150, 64, dtype, True, 0, 0, -0.2, seed=6, label="negative scale")
    _bwd_case(1, 2, 2, 150, 64, dtype, False, 0, 0, 0.0, seed=7, label="zero scale")
    # a window wide enough that a key block sees masked, then fully visible,
    # then masked query blocks, repeated over the query heads of each group
    _bwd_case(1, 4, 2, 700, 128, dtype, True, 300, 4, 0.088, seed=8, label="gqa window")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_sharp_softmax(dtype, dkv_kernel):
    """Q x 6: nearly one-hot probability rows, so P is recomputed from scores far
    from the row max (exp2 arguments down to about -100) and dS is dominated by
    a few keys per row."""
    q, k, v = fa_inputs.make_qkv(1, 2, 300, 128, dtype, seed=21)
    q6 = (q.float() * 6).to(q.dtype)
    dout = fa_inputs.make_qkv(1, 2, 300, 128, dtype, seed=22)[0]
    scale = 1.0 / math.sqrt(128)
    qd, kd, vd = (t.cuda() for t in (q6, k, v))
    o, lse = fa.flash_attn_fwd(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = fa.flash_attn_bwd(qd, kd, vd, o, lse, dout.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = ORACLE.attention_bwd(fa_inputs.to_f64(q6), fa_inputs.to_f64(k), fa_inputs.to_f64(v),
                                      fa_inputs.to_f64(dout), causal=True, scale=scale)
    errs = [_grad_err(dq, rq), _grad_err(dk, rk), _grad_err(dv, rv)]
    _say(f"  {dtype} Qx6 backward: dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    assert max(errs) <= TOL_G[dtype], errs


def test_split_keys_sharp_softmax():
    """Key splits on nearly one-hot rows: partial LSEs of one row differ by tens,
    and the merge must weight the partials by them (not average them)."""
    q, k, v = fa_inputs.make_qkv(1, 2, 700, 128, "bf16", seed=23)
    q8 = (q.float() * 8).to(q.dtype)
    for n_split in (2, 5):
        o, lse = fa.flash_attn_fwd_split(q8.cuda(), k.cuda(), v.cuda(), n_split=n_split,
                                         causal=True, scale=1 / math.sqrt(128))
        torch.cuda.synchronize()
        compare(o, lse, q8, k, v, "bf16", causal=True, scale=1 / math.sqrt(128),
                label=f"bf16 Qx8 split{n_split}")


def test_backward_headline_shape_sampled(dkv_kernel):
    """The headline shape (B4 H16 S4096 D128 bf16 causal): two heads against
    the oracle, the rest finite."""
    B, H, S, D = 4, 16, 4096, 128
    q, k, v = fa_inputs.make_qkv(B, H, S, D, "bf16", seed=0)
    dout, _, _ = fa_inputs.make_qkv(B, H, S, D, "bf16", seed=9)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.flash_attn_fwd(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = fa.flash_attn_bwd(qd, kd, vd, o, lse, dod, causal=True, scale=scale)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b, h in [(0, 0), (3, 15)]:
        rq, rk, rv = ORACLE.attention_bwd(
            fa_inputs.to_f64(q[b:b + 1, h:h + 1]), fa_inputs.to_f64(k[b:b + 1, h:h + 1]),
            fa_inputs.to_f64(v[b:b + 1, h:h + 1]), fa_inputs.to_f64(dout[b:b + 1, h:h + 1]),
            causal=True, scale=scale)
        errs = [_grad_err(g[b:b + 1, h:h + 1], r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
        _say(f"  headline head ({b},{h}): dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
        assert max(errs) <= TOL_G["bf16"]
