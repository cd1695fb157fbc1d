"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one forward pass (both contractions, online softmax, epilogue) over
the whole batch of the workload, inputs already resident in HBM. Prints ONE
JSON line. Throughput is TFLOP/s with FLOPs = 4*B*H*S^2*D, halved under the
causal mask; under a sliding window (+ sinks) FLOPs = 4*B*H*D*(kept query-key
pairs), since the nominal causal figure would count the keys the window drops
(it is reported beside it in `config`).

`roofline` describes the forward kernel: achieved = algorithmic FLOPs of one
launch / mean launch duration (HIP events on the stream the kernel runs on);
peak = MI355X dense bf16/fp16 MFMA (2516.6 TFLOP/s = 256 CU x 2.4 GHz x 4096
FLOP/clk) or fp32 MFMA (157.3 TFLOP/s); traffic = counter-measured HBM bytes
per launch when the kernel sources match those the counters were taken on,
else null. `cpu_baseline` times the fp64 CPU oracle on a bounded sample of the
same workload (whole heads, all rows, sized to ~20 s).
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

# HBM bytes per step measured with rocprofv3 counter runs (FETCH_SIZE scaled
# x2.0 and WRITE_SIZE x1.0, the factors a 256 MiB device copy of known size
# gives), keyed by workload and the SHA-256 of the kernel sources the counters
# were taken on. Any other source tree reports traffic = null.
FWD_SOURCES = ["io_aware_tiled_flash_amd/csrc/fa_fwd_fast.hip",
               "io_aware_tiled_flash_amd/csrc/fa_device.h",
               "io_aware_tiled_flash_amd/csrc/fa_kernel.h",
               "io_aware_tiled_flash_amd/csrc/fa_lds.h"]
BWD_SOURCES = ["io_aware_tiled_flash_amd/csrc/fa_bwd.hip",
               "io_aware_tiled_flash_amd/csrc/fa_device.h",
               "io_aware_tiled_flash_amd/csrc/fa_kernel.h",
               "io_aware_tiled_flash_amd/csrc/fa_lds.h"]
MEASURED_TRAFFIC = {
    # forward kernel, 4 waves: FETCH 389972.4 KiB, WRITE 66878.1 KiB per launch
    ("causal_b4h16s4096d128_bf16",
     "1f643d292e14bd72dd1eea47422a89db1e7a702035ffeb313375880610382494"): 867146650,
    # dq + dkv kernels: FETCH 428291.4 + 364639.4 KiB, WRITE 67618.7 + 131072.3 KiB per step
    ("bwd_causal_b4h16s4096d128_bf16",
     "86faa674d37e18ea9f12a83052f8d7abcf34ed54ba35d0139e6681acc98fa52f"): 1827381862,
    # forward kernel, f16 D=64: FETCH 3204.8 KiB, WRITE 2112 KiB per launch
    ("noncausal_b2h8s1024d64_f16",
     "1f643d292e14bd72dd1eea47422a89db1e7a702035ffeb313375880610382494"): 8726118,
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
    # The board takes on the order of a hundred back-to-back launches of the
    # headline shape (~30 ms of load) to leave its idle power state: the
    # first 20 launches run ~20 % slower than the steady state.
    ap.add_argument("--warmup", type=int, default=150)
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
    if w.backward:
        return f"fa::fa_bwd_dq_kernel + fa::fa_bwd_dkv_kernel <{w.dtype},D={w.D}> (128-row / 128-key tiles)"
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[w.dtype]
    bq, bk = fa.flash_attn_tile_shape(w.B, w.H, w.S, w.D, code)
    if w.dtype != "f32" and w.D in (64, 128):
        return f"fa::fa_fwd_fast_kernel<{w.dtype},D={w.D},waves={bq // 32}> ({bq}x{bk} tile)"
    return f"fa::fa_fwd_{'f32' if w.dtype == 'f32' else 'half'}_kernel<D={w.D}> ({bq}x{bk} tile)"


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


def cpu_baseline(w, q, k, v, n_heads: int, budget_s: float = 20.0):
    """Time the fp64 oracle on the first n_heads (b, h) heads, all rows. With
    n_heads = 0 the sample is sized from one timed head to about budget_s seconds
    (capped at the whole workload)."""
    import numpy as np
    from oracle import attention as oracle
    import fa_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = 1
    all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    G = w.H // w.kv_heads
    slopes = alibi_slopes(w.H) if w.alibi else None
    dout = fa_inputs.make_dout(w) if w.backward else None

    def head(b, h):
        g = h // G
        return (fa_inputs.to_f64(q[b:b + 1, h:h + 1]), fa_inputs.to_f64(k[b:b + 1, g:g + 1]),
                fa_inputs.to_f64(v[b:b + 1, g:g + 1]), None if slopes is None else [slopes[h]])

    def run(arrs):
        t0 = time.perf_counter()
        for n_, (qq, kk, vv, sl) in enumerate(arrs):
            if w.backward:
                b, h = all_heads[n_]
                oracle.attention_bwd(qq, kk, vv, fa_inputs.to_f64(dout[b:b + 1, h:h + 1]),
                                     causal=w.causal, scale=w.scale, window=w.window,
                                     n_sink=w.n_sink, alibi_slopes=sl)
            else:
                oracle.attention_fwd(qq, kk, vv, causal=w.causal, scale=w.scale,
                                     window=w.window, n_sink=w.n_sink, alibi_slopes=sl)
        return time.perf_counter() - t0

    if n_heads <= 0:
        run([head(*all_heads[0])])                  # first call warms the BLAS threads
        t_one = run([head(*all_heads[0])])
        n_heads = max(1, min(len(all_heads), int(budget_s / max(t_one, 1e-3))))
    heads = all_heads[:n_heads]
    dt = run([head(b, h) for b, h in heads])
    flops = work_flops(w) * len(heads) / (w.B * w.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(heads)} of {w.B * w.H} heads (all {w.S} rows each) of the same "
                      f"workload, fp64 NumPy, {dt:.2f} s wall"}


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
    import io_aware_tiled_flash_amd as fa

    name = args.workload or fa_inputs.HEADLINE
    w = fa_inputs.ALL_WORKLOADS[name]
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    q, k, v = fa_inputs.make_workload(w)
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
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": MEASURED_TRAFFIC.get((name, kernel_source_hash(w.backward))),  # bytes per step
                     "kernel": kernel_name(fa, w),
                     "mean_launch_us": round(mean_launch_ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_sample_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
