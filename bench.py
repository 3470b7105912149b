"""Benchmark: exact attention forward + backward on one MI355X.

A step is one pass of the whole hot path over one batch: fa2_fwd then fa2_bwd
(delta pass, key-block pass, dQ conversion) on the causal N=8192, d=128 bf16
workload (B=4, H=32), inputs resident in HBM. FLOPs follow the convention
of the workload definition: forward 4*B*H*N^2*d, halved for causal; backward
2.5x forward. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "attention fwd/bwd TFLOP/s and % of MI355X bf16 MFMA peak, N=8k d=128 causal"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def flops(B, H, N, d, causal):
    fwd = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    return fwd, 2.5 * fwd


def cpu_baseline(w, min_seconds=10.0, max_heads=16):
    """The fp64 oracle (as it stands) on a bounded sample: full forward + backward of
    single (b, h) heads of the workload, one after another, until about `min_seconds`
    of CPU work (at most `max_heads`), in the same FLOP convention."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    heads = 0
    sec = 0.0
    while heads < max_heads and (heads == 0 or sec < min_seconds):
        t = workloads.make_inputs(1, 1, w.N, w.d, "bf16", seed=w.number * 1000 + heads, with_dout=True)
        start = time.perf_counter()
        oracle.attention_forward(t["q"], t["k"], t["v"], w.scale, w.causal, w.window)
        oracle.attention_backward(t["q"], t["k"], t["v"], t["dout"], w.scale, w.causal, w.window)
        sec += time.perf_counter() - start
        heads += 1
    f_fwd, f_bwd = flops(1, heads, w.N, w.d, w.causal)
    return {
        "value": (f_fwd + f_bwd) / sec / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} (b,h) heads, full fp64 forward+backward at N={w.N}, d={w.d}, "
                  f"causal; {sec:.2f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 launches), used to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters against a known byte count")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path shards by "
              f"(batch, head) with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return

    import exact_tiled_attention_06_amd as fa2
    import workloads

    fa2.load_library()
    w = workloads.WORKLOADS[3]  # B=4, H=32, N=8192, d=128, causal
    B, H, N, d = w.B, w.H, w.N, w.d
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=w.number, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    del t
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["dout"]
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa2.fa2_bwd_workspace_size(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    scale = w.scale
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    det = int(args.deterministic)

    def fwd():
        fa2.fa2_fwd(q, k, v, out, lse, B, H, N, d, scale, 1, -1, -1, None, sp)

    def bwd():
        fa2.fa2_bwd(q, k, v, out, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, scale, 1, -1, -1, None, det, sp)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    fwd_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    bwd_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    ms_step = total_ms / K
    f_fwd, f_bwd = flops(B, H, N, d, True)
    fwd_avg = sum(fwd_ms) / K
    bwd_avg = sum(bwd_ms) / K
    fwd_tf = f_fwd / (fwd_avg * 1e-3) / 1e12
    bwd_tf = f_bwd / (bwd_avg * 1e-3) / 1e12
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    kernels = {
        "fa2_fwd": {"kernel": "fwd_bf16_kernel<128,4,64>", "bound": "mfma", "achieved": round(fwd_tf, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                    "avg_ms": round(fwd_avg, 4), "median_ms": round(fwd_ms[K // 2], 4),
                    "flop_per_launch": f_fwd},
        "fa2_bwd": {"kernel": "bwd_main_kernel<128> (+ delta and dQ-convert passes in the same call)",
                    "bound": "mfma", "achieved": round(bwd_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4), "avg_ms": round(bwd_avg, 4),
                    "median_ms": round(bwd_ms[K // 2], 4), "flop_per_launch": f_bwd},
    }
    dom = "fa2_bwd" if bwd_avg >= fwd_avg else "fa2_fwd"
    dk_ = kernels[dom]
    roofline = {"bound": "mfma", "achieved": dk_["achieved"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": dk_["frac"], "traffic": None, "kernel": dk_["kernel"], "call": dom}

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 causal attention fwd+bwd, B=4 H=32 N=8192 d=128 [B,N,H,d]",
                   "B": B, "H": H, "N": N, "d": d, "causal": True, "seq_len": N, "global_batch": B,
                   "parallelism": "none (1 GPU)", "deterministic_bwd": bool(det)},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
