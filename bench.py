"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-s T] [--workload NAME]
                    [--no-cpu-baseline]

One step = one forward pass (both contractions, online softmax, epilogue) over
the whole batch of the workload, inputs already resident in HBM. Prints ONE
JSON line. Throughput is TFLOP/s with FLOPs = 4*B*H*S^2*D, halved under the
causal mask; under a sliding window (+ sinks) FLOPs = 4*B*H*D*(kept query-key
pairs), since the nominal causal figure would count the keys the window drops
(it is reported beside it in `config`).

Timing protocol: `prewarm` seconds of untimed launches (reported as their own
field: the board takes about a hundred launches of the headline shape to leave
its idle clocks), then exactly `warmup` untimed launches, then exactly `steps`
launches between one pair of HIP events on the launch stream, with
torch.cuda.synchronize() on both sides. After the timed region an untimed pass
of up to 50 launches with an event pair each gives the per-launch spread
(min / median / p90).

`roofline` describes the forward kernel: achieved = algorithmic FLOPs of one
launch / mean launch duration of the timed region; peak = MI355X dense
bf16/fp16 MFMA (2516.6 TFLOP/s = 256 CU x 2.4 GHz x 4096 FLOP/clk) or fp32
MFMA (157.3 TFLOP/s); traffic = counter-measured HBM bytes per launch when the
launched kernel (wave count, key parts) and its sources match those the
counters were taken on, else null.

`cpu_baseline` times the fp64 CPU oracle on the same inputs: whole heads (all
rows), fanned out over a process pool of one single-threaded worker per host
core available to this process (at most 16), started before the GPU is
touched. `parity` compares the GPU result of the timed launches with that
oracle output on every head the baseline ran: max|dO| and the LSE error
against the stated tolerances (for the backward workload, the normwise
gradient errors).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
TOL_O = {"f32": 1e-5, "f16": 4e-3, "bf16": 1.6e-2}
TOL_LSE_REL = 1e-3
TOL_GRAD = {"f16": 4e-3, "bf16": 2.5e-2}
MAX_POOL = 16

# HBM bytes per step measured with rocprofv3 counter runs (FETCH_SIZE scaled
# x2.0 and WRITE_SIZE x1.0, the factors a 256 MiB device copy of known size
# gives), keyed by workload, the kernel the host plan launches for it (wave
# count, key parts) and the SHA-256 of the kernel sources the counters were
# taken on. Any other plan or source tree reports traffic = null.
FWD_SOURCES = ["io_aware_tiled_flash_amd/csrc/fa_fwd_fast.hip",
               "io_aware_tiled_flash_amd/csrc/fa_device.h",
               "io_aware_tiled_flash_amd/csrc/fa_shapes.h",
               "io_aware_tiled_flash_amd/csrc/fa_lds.h"]
BWD_SOURCES = ["io_aware_tiled_flash_amd/csrc/fa_bwd.hip",
               "io_aware_tiled_flash_amd/csrc/fa_device.h",
               "io_aware_tiled_flash_amd/csrc/fa_shapes.h",
               "io_aware_tiled_flash_amd/csrc/fa_lds.h"]
MEASURED_TRAFFIC: dict = {
    ("causal_b4h16s4096d128_bf16",
     "fa::fa_fwd_fast_kernel<bf16,D=128,waves=8> (256x64 tile)",
     "cf0e7cd960b9e263fa05a241594851d179c68273fd52a28df40389910730ad31"): 373837414,
    ("causal_b1h32s16384d128_bf16",
     "fa::fa_fwd_fast_kernel<bf16,D=128,waves=8> (256x64 tile)",
     "cf0e7cd960b9e263fa05a241594851d179c68273fd52a28df40389910730ad31"): 1672267162,
    ("window1024_sink4_b8h32s8192d128_bf16",
     "fa::fa_fwd_fast_kernel<bf16,D=128,waves=4> (128x64 tile)",
     "cf0e7cd960b9e263fa05a241594851d179c68273fd52a28df40389910730ad31"): 2246306202,
    ("noncausal_b2h8s1024d64_f16",
     "fa::fa_fwd_parts_kernel<f16,D=64,parts=4> (8 waves, 64x64 tile)",
     "cf0e7cd960b9e263fa05a241594851d179c68273fd52a28df40389910730ad31"): 9184870,
    ("bwd_causal_b4h16s4096d128_bf16",
     "fa::fa_bwd_dq_kernel<bf16,D=128> (128 rows, 4 waves) + fa_bwd_dkv2_kernel<bf16,D=128> (128 keys, 4 waves, 2 work-groups per CU)",
     "35da84e324f63fb02051f45a7017d6980165b754c353cb789df7ae33507e3385"): 1227915059,
}


def kernel_source_hash(backward: bool = False) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in (BWD_SOURCES if backward else FWD_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed launches before the warm-up (reported)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=0,
                    help="heads of the workload the oracle baseline runs (0 = auto)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB, --steps times "
                         "(calibrates the HBM byte counters against a known size)")
    return ap.parse_args()


def copy_probe(mib: int, steps: int):
    """Device-to-device copies of `mib` MiB, each preceded by writing a 1 GiB
    buffer so that the source is no longer held in L2 / Infinity Cache."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    flush = torch.empty((1 << 30) // 4, dtype=torch.float32, device="cuda")
    for _ in range(steps):
        flush.fill_(1.0)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read_per_launch": n * 4,
                      "copy_probe_bytes_written_per_launch": n * 4, "launches": steps}))


def kernel_name(fa, w) -> str:
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[w.dtype]
    if w.backward:
        return "fa::" + fa.flash_attn_bwd_kernel(w.B, w.H, w.S, w.D, code, H_kv=w.kv_heads,
                                                 causal=w.causal, window=w.window, alibi=w.alibi)
    return "fa::" + fa.flash_attn_fwd_kernel(w.B, w.H, w.S, w.D, code, alibi=w.alibi,
                                             n_split=w.n_split, window=w.window)


def nominal_flops(w) -> float:
    """4*B*H*S^2*D, halved under the causal mask."""
    f = 4.0 * w.B * w.H * w.S * w.S * w.D
    return f / 2.0 if w.causal else f


def work_flops(w) -> float:
    """FLOPs of one step: the forward's algorithmic FLOPs, or for a backward
    workload 2.5 times them (five S x S x D products -- S, dP, dV, dQ, dK --
    against the forward's two)."""
    return algorithmic_flops(w) * (2.5 if w.backward else 1.0)


def algorithmic_flops(w) -> float:
    """FLOPs of the two contractions over the (query, key) pairs the mask keeps.
    Equal to the nominal figure up to the causal diagonal; under a sliding window
    the nominal causal figure would count keys the window drops."""
    if w.causal and 0 < w.window < w.S:
        return 4.0 * w.B * w.H * w.D * kept_pairs(w)
    return nominal_flops(w)


def kept_pairs(w) -> int:
    S, W, ns = w.S, w.window, w.n_sink
    if not w.causal:
        return S * S
    if W == 0 or W >= S:
        return S * (S + 1) // 2
    tot = W * (W + 1) // 2 + (S - W) * W
    tot += sum(min(ns, i - W + 1) for i in range(W, S))
    return tot


def alibi_slopes(H: int):
    """Per-head ALiBi slopes of the Lesson 91 deck (slide 23): 2^(-8h/H), h = 1..H."""
    return [2.0 ** (-8.0 * h / H) for h in range(1, H + 1)]


# --------------------------------------------------------------------------- #
# CPU baseline: the oracle on a process pool (no GPU is touched by this leg).
# --------------------------------------------------------------------------- #

def _limit_blas():
    """Pool initializer: one BLAS thread per worker (set before numpy loads)."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_head(job):
    """One (b, h) head of the workload through the oracle: (O, LSE) of the
    forward, or (dQ, dK, dV) of the backward, for the head's inputs (float32
    arrays holding the stored values exactly)."""
    from oracle import attention as oracle
    qh, kh, vh, dh, slope, kw, backward = job
    t0 = time.perf_counter()
    if backward:
        res = oracle.attention_bwd(qh, kh, vh, dh, alibi_slopes=slope, **kw)
    else:
        res = oracle.attention_fwd(qh, kh, vh, alibi_slopes=slope, **kw)
    return res, time.perf_counter() - t0


def _host_info():
    info = {"affinity_cores": len(os.sched_getaffinity(0))}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import numpy as np
    info["numpy"] = np.__version__
    try:
        from threadpoolctl import threadpool_info
        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:
        pass
    return info


def cpu_baseline(w, q, k, v, n_heads: int, budget_s: float = 20.0):
    """Time the fp64 oracle on whole heads of the workload (all rows), one
    head per task over a pool of single-threaded workers. With n_heads = 0 the
    sample is every head, cut down to about budget_s seconds of wall time from
    the time of the first round of heads. Returns (baseline record, the heads
    run, their oracle results)."""
    import multiprocessing as mp
    import numpy as np
    import fa_inputs
    all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    G = w.H // w.kv_heads
    slopes = alibi_slopes(w.H) if w.alibi else None
    dout = fa_inputs.make_dout(w) if w.backward else None
    kw = dict(causal=w.causal, scale=w.scale, window=w.window, n_sink=w.n_sink)
    f32 = lambda t: t.float().numpy()   # exact for bf16 / f16 / f32 values

    def job(b, h):
        g = h // G
        return (f32(q[b:b + 1, h:h + 1]), f32(k[b:b + 1, g:g + 1]), f32(v[b:b + 1, g:g + 1]),
                None if dout is None else f32(dout[b:b + 1, h:h + 1]),
                None if slopes is None else [slopes[h]], kw, w.backward)

    n_proc = max(1, min(MAX_POOL, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")     # fresh interpreters: nothing of this process is inherited
    with ctx.Pool(n_proc, initializer=_limit_blas) as pool:
        pool.map(_limit_blas_probe, range(n_proc))       # workers up and imported
        if n_heads <= 0:
            first = all_heads[:n_proc]
            t0 = time.perf_counter()
            res0 = pool.map(_oracle_head, [job(*bh) for bh in first])
            t_round = time.perf_counter() - t0
            rounds = max(1, int(budget_s / max(t_round, 1e-3)))
            n_heads = min(len(all_heads), rounds * n_proc)
            rest = all_heads[len(first):n_heads]
            t0 = time.perf_counter()
            res1 = pool.map(_oracle_head, [job(*bh) for bh in rest]) if rest else []
            dt = t_round + (time.perf_counter() - t0)
            heads = all_heads[:max(n_heads, len(first))]
            results = [r for r, _ in res0 + res1]
        else:
            heads = all_heads[:n_heads]
            t0 = time.perf_counter()
            results = [r for r, _ in pool.map(_oracle_head, [job(*bh) for bh in heads])]
            dt = time.perf_counter() - t0
    flops = work_flops(w) * len(heads) / (w.B * w.H)
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": n_proc, "kind": "oracle",
           "sample": f"{len(heads)} of {w.B * w.H} heads (all {w.S} rows each) of the same "
                     f"workload, fp64 NumPy, {n_proc} single-threaded worker processes, "
                     f"{dt:.2f} s wall",
           "blas_threads_per_worker": 1, **_host_info()}
    return rec, heads, results


def _limit_blas_probe(_):
    import numpy  # noqa: F401
    from oracle import attention  # noqa: F401
    return os.getpid()


def parity(w, heads, results, gpu_out):
    """GPU results against the oracle on the heads the baseline ran."""
    import numpy as np
    if w.backward:
        dq, dk, dv = (t.float().cpu().double().numpy() for t in gpu_out)
        G = w.H // w.kv_heads
        worst = [0.0, 0.0, 0.0]
        # dK, dV of a key/value head sum over its query group: compare them only
        # when the sample holds every query head of the group
        for (b, h), (rq, rk, rv) in zip(heads, results):
            worst[0] = max(worst[0], float(np.abs(dq[b, h] - rq[0, 0]).max() /
                                           max(1.0, np.abs(rq[0, 0]).max())))
            if G == 1:
                for n, (gt, rt) in enumerate(((dk, rk), (dv, rv)), start=1):
                    worst[n] = max(worst[n], float(np.abs(gt[b, h] - rt[0, 0]).max() /
                                                   max(1.0, np.abs(rt[0, 0]).max())))
        tol = TOL_GRAD[w.dtype]
        return {"heads": len(heads), "rows_per_head": w.S, "normwise_dq": worst[0],
                "normwise_dk": worst[1], "normwise_dv": worst[2], "tol": tol,
                "pass": bool(max(worst) <= tol)}
    o, lse = gpu_out
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    d_o, d_l = 0.0, 0.0
    for (b, h), (O, L) in zip(heads, results):
        d_o = max(d_o, float(np.abs(og[b, h] - O[0, 0]).max()))
        d_l = max(d_l, float((np.abs(lg[b, h] - L[0, 0]) / np.maximum(1.0, np.abs(L[0, 0]))).max()))
    tol_o = TOL_O[w.dtype]
    return {"heads": len(heads), "rows_per_head": w.S, "max_abs_dO": d_o, "tol_O": tol_o,
            "max_rel_dLSE": d_l, "tol_LSE_rel": TOL_LSE_REL,
            "pass": bool(d_o <= tol_o and d_l <= TOL_LSE_REL)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward pass here runs on a single "
              "MI355X (the multi-GPU sharding is a design note, not built); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps)
        return

    import torch
    import fa_inputs

    name = args.workload or fa_inputs.HEADLINE
    w = fa_inputs.ALL_WORKLOADS[name]
    q, k, v = fa_inputs.make_workload(w)

    # The oracle leg runs first, before anything touches the GPU, so that its
    # worker processes start from a process with no GPU state.
    base, heads, oracle_res = None, None, None
    if not args.no_cpu_baseline:
        base, heads, oracle_res = cpu_baseline(w, q, k, v, args.cpu_sample_heads)

    import io_aware_tiled_flash_amd as fa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    slopes = (torch.tensor(alibi_slopes(w.H), dtype=torch.float32, device=dev)
              if w.alibi else None)

    dout = fa_inputs.make_dout(w).to(dev) if w.backward else None
    if w.backward:
        o_f, lse_f = fa.flash_attn_fwd(qd, kd, vd, causal=w.causal, window=w.window,
                                       n_sink=w.n_sink, scale=w.scale, alibi_slopes=slopes)
        bws = torch.empty(fa.flash_attn_bwd_workspace_bytes(w.B, w.H, w.S), dtype=torch.uint8,
                          device=dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = None
    if w.n_split > 1:
        ws = torch.empty(fa.flash_attn_split_workspace_bytes(w.B, w.H, w.S, w.D, w.n_split),
                         dtype=torch.uint8, device=dev)

    def step():
        if w.backward:
            fa.flash_attn_bwd(qd, kd, vd, o_f, lse_f, dout, causal=w.causal, window=w.window,
                              n_sink=w.n_sink, scale=w.scale, alibi_slopes=slopes,
                              workspace=bws, dq=dq, dk=dk, dv=dv)
        elif w.n_split > 1:
            fa.flash_attn_fwd_split(qd, kd, vd, n_split=w.n_split, causal=w.causal,
                                    window=w.window, n_sink=w.n_sink, scale=w.scale,
                                    alibi_slopes=slopes, workspace=ws, out=o, lse=lse)
        else:
            fa.flash_attn_fwd(qd, kd, vd, causal=w.causal, window=w.window, n_sink=w.n_sink,
                              scale=w.scale, alibi_slopes=slopes, out=o, lse=lse)

    # Pre-warm: untimed launches for prewarm_s seconds (queue at most 32 ahead).
    prewarm_n = 0
    torch.cuda.synchronize()
    t_pw = time.perf_counter()
    while time.perf_counter() - t_pw < args.prewarm_s:
        for _ in range(8):
            step()
        prewarm_n += 8
        if prewarm_n % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    prewarm_s = time.perf_counter() - t_pw if prewarm_n else 0.0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # One HIP event pair on the launch stream brackets the K steps: an event
    # pair per step would put two more packets between kernels and, for the
    # short shapes, stretch the gap between launches.
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_ms = start.elapsed_time(end) / args.steps
    gpu_out = (dq, dk, dv) if w.backward else (o, lse)
    gpu_out = tuple(t.clone() for t in gpu_out)

    # Untimed pass: one event pair per launch, for the spread.
    n_stat = min(args.steps, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_stat)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)

    def pct(p):
        return per[min(len(per) - 1, int(math.ceil(p / 100.0 * len(per))) - 1)]

    flops = work_flops(w)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / (mean_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    e = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    alg_bytes = (2 * w.H + 2 * w.kv_heads) * w.B * w.S * w.D * e + 4 * w.B * w.H * w.S
    if w.backward:   # reads q, k, v, o, dO, lse; writes dq, dk, dv
        alg_bytes = (4 * w.H + 4 * w.kv_heads) * w.B * w.S * w.D * e + 4 * w.B * w.H * w.S

    out = {
        "metric": "attention fwd TFLOP/s & % MFMA peak (causal bf16 B4 H16 S4096 D128)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: Q, K, V iid N(0,1), numpy default_rng(seed 0), rounded to dtype",
        "config": {"workload": name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "S": w.S, "D": w.D,
                   "alibi": w.alibi, "n_split": w.n_split, "backward": w.backward,
                   "causal": w.causal, "window": w.window, "n_sink": w.n_sink,
                   "scale": w.scale, "layout": "[B,H,S,D] contiguous",
                   "flops_per_step": flops, "nominal_flops_per_step": nominal_flops(w),
                   "kept_pairs_per_head": kept_pairs(w),
                   "frac_of_peak_wall": round(value / peak, 4),
                   "alg_hbm_bytes_per_step": alg_bytes,
                   "alg_hbm_GBps": round(alg_bytes / (mean_launch_ms * 1e-3) / 1e9, 1)},
        "prewarm": {"seconds": round(prewarm_s, 3), "launches": prewarm_n},
        "launch_us": {"passes": n_stat, "min": round(per[0], 2), "median": round(pct(50), 2),
                      "p90": round(pct(90), 2), "max": round(per[-1], 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": MEASURED_TRAFFIC.get((name, kernel_name(fa, w),
                                                      kernel_source_hash(w.backward))),
                     "kernel": kernel_name(fa, w),
                     "mean_launch_us": round(mean_launch_ms * 1e3, 2)},
        "cpu_baseline": base,
        "parity": None if base is None else parity(w, heads, oracle_res, gpu_out),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
