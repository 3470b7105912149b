"""Benchmark: exact attention forward + backward on one MI355X.

A step is one pass of the whole hot path over one batch: fa2_fwd then the
backward's two passes (the dQ pass, which also forms D = rowsum(dO*O) and the
per-row values, then the dK/dV pass; exactly what fa2_bwd runs) on the causal
N=8192, d=128 bf16 workload (B=4, H=32), inputs
resident in HBM. FLOPs follow the convention of the workload definition:
forward 4*B*H*N^2*d, halved for causal; backward 2.5x forward. Prints ONE JSON
line.

After the timed steps, the packed variable-length workload (32768 tokens in 12
ragged sequences, H=32, d=128, causal) is timed the same way through
fa2_fwd_varlen / fa2_bwd_varlen and reported under "varlen", with the FLOP
convention applied per sequence. Then the block-sparse workload (the same
B=4, H=32, N=8192, d=128 causal shape with a 128 x 128 block mask: a band of
width 1 around the diagonal, one global key block and 10 % random blocks,
about 18 % of the causal blocks) is timed through fa2_fwd_blocksparse /
fa2_bwd_blocksparse and reported under "blocksparse", counting the visible
(query, key) pairs of the active blocks. Last, the dense causal workload with
dropout p = 0.1 on the attention weights (keep matrix from Philox4x32-10,
regenerated in the backward) is timed through fa2_fwd_dropout /
fa2_bwd_dropout and reported under "dropout", with the dense FLOP convention.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-varlen] [--no-sparse]
                  [--no-dropout]
  python bench.py --other-workloads   # the other dense workloads (d=64 non-causal, N=4096 causal,
                                      # N=16384 window + ALiBi), one JSON line, not the headline
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
    host = host_info()
    return {
        "value": (f_fwd + f_bwd) / sec / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} (b,h) heads, full fp64 forward+backward at N={w.N}, d={w.d}, "
                  f"causal; {sec:.2f} s measured; the whole workload would take about "
                  f"{sec * w.B * w.H / heads:.0f} s at this rate (extrapolated)",
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": host["cpu_model"],
        "blas": host["blas"],
        "blas_threads": blas_threads,
    }


def host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS library numpy calls, with its threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({os.path.basename(i.get('filepath', ''))})"
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def phase_stats(samples):
    """Mean, median and min of a list of per-step milliseconds."""
    xs = sorted(samples)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"avg_ms": sum(xs) / n, "median_ms": med, "min_ms": xs[0]}


def timed_stats(phases, steps, warmup, stream):
    """Per-step milliseconds of each (name, fn) phase, HIP events recorded on `stream`
    (the stream the kernels are launched on) around every launch; returns
    {name: {avg_ms, median_ms, min_ms}}."""
    import torch
    for _ in range(warmup):
        for _, fn in phases:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for n, (_, fn) in enumerate(phases):
            fn()
            ev[i][n + 1].record(stream)
    torch.cuda.synchronize()
    return {name: phase_stats([e[n].elapsed_time(e[n + 1]) for e in ev]) for n, (name, _) in enumerate(phases)}


def timed(phases, steps, warmup, stream):
    """Average milliseconds of each (name, fn) phase over `steps` passes, HIP events on `stream`."""
    return {k: v["avg_ms"] for k, v in timed_stats(phases, steps, warmup, stream).items()}


def bench_varlen(fa2, workloads, steps, warmup):
    """Packed variable-length workload: fa2_fwd_varlen + fa2_bwd_varlen, timed with events."""
    import torch
    w = workloads.VARLEN_WORKLOADS[6]
    t = workloads.varlen_workload_inputs(w)
    lengths = [int(x) for x in t["lengths"]]
    T, H, d = w.total, w.H, w.d
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "dout"))
    cu = t["cu_seqlens"].cuda()
    out = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa2.fa2_bwd_workspace_size(1, H, T, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    causal = int(w.causal)

    def fwd():
        fa2.fa2_fwd_varlen(q, k, v, out, lse, cu, w.nseq, T, H, d, w.scale, causal, -1, -1, None, sp)

    def bwd():
        fa2.fa2_bwd_varlen(q, k, v, out, lse, do, dq, dk, dv, cu, ws, ws_bytes, w.nseq, T, H, d, w.scale, causal,
                           -1, -1, None, sp)

    ms = timed([("fwd", fwd), ("bwd", bwd)], steps, warmup, stream)
    f_fwd = sum(flops(1, H, n, d, w.causal)[0] for n in lengths)
    f_bwd = 2.5 * f_fwd
    fwd_tf = f_fwd / (ms["fwd"] * 1e-3) / 1e12
    bwd_tf = f_bwd / (ms["bwd"] * 1e-3) / 1e12
    step_tf = (f_fwd + f_bwd) / ((ms["fwd"] + ms["bwd"]) * 1e-3) / 1e12
    return {
        "workload": f"bf16 packed causal attention fwd+bwd, T={T} tokens in {w.nseq} sequences, H={H} d={d}",
        "lengths": lengths,
        "fwd_ms": round(ms["fwd"], 4),
        "bwd_ms": round(ms["bwd"], 4),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "tflops": round(step_tf, 2),
        "frac_of_peak": round(step_tf / PEAK_BF16_TFLOPS, 4),
        "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "flop_convention": "per sequence: forward 4*H*n^2*d/2 (causal), backward 2.5x",
    }


def causal_block_pairs(N, block=128):
    """[nb, nb] number of causal-visible (query, key) pairs in each block pair."""
    import numpy as np
    nb = -(-N // block)
    out = np.zeros((nb, nb))
    for r in range(nb):
        i = np.arange(r * block, min(N, r * block + block))
        for c in range(r + 1):
            s, e = c * block, min(N, c * block + block)
            out[r, c] = np.clip(i - s + 1, 0, e - s).sum()
    return out


def bench_blocksparse(fa2, workloads, steps, warmup):
    """Block-sparse workload: fa2_fwd_blocksparse + fa2_bwd_blocksparse, timed with events.
    FLOPs: 4*d per visible pair of the active blocks (forward), 2.5x that (backward)."""
    import torch
    w = workloads.SPARSE_WORKLOADS[7]
    B, H, N, d = w.B, w.H, w.N, w.d
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=w.number, with_dout=True)
    mask = workloads.sparse_block_mask(H, N, w.local, w.global_blocks, w.density, seed=w.number)
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "dout"))
    del t
    m = mask.cuda()
    nb = m.shape[-1]
    sh = nb * nb  # [1, H, nb, nb]: shared across the batch
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa2.fa2_bwd_workspace_size(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def fwd():
        fa2.fa2_fwd_blocksparse(q, k, v, out, lse, B, H, N, d, w.scale, 1, -1, -1, None, m, 0, sh, sp)

    def bwd():
        fa2.fa2_bwd_blocksparse(q, k, v, out, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, w.scale, 1, -1, -1, None,
                                m, 0, sh, sp)

    ms = timed([("fwd", fwd), ("bwd", bwd)], steps, warmup, stream)
    per_block = causal_block_pairs(N)
    active = mask[0].numpy().astype(bool)
    pairs = B * float((per_block[None] * active).sum())
    dense_pairs = B * H * float(per_block.sum())
    f_fwd = 4.0 * d * pairs
    f_bwd = 2.5 * f_fwd
    fwd_tf = f_fwd / (ms["fwd"] * 1e-3) / 1e12
    bwd_tf = f_bwd / (ms["bwd"] * 1e-3) / 1e12
    step_ms = ms["fwd"] + ms["bwd"]
    step_tf = (f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12
    return {
        "workload": (f"bf16 block-sparse causal attention fwd+bwd, B={B} H={H} N={N} d={d}, 128x128 block mask: "
                     f"band {w.local}, {w.global_blocks} global block, {w.density:.0%} random (seeded per head)"),
        "active_pair_fraction": round(pairs / dense_pairs, 4),
        "fwd_ms": round(ms["fwd"], 4),
        "bwd_ms": round(ms["bwd"], 4),
        "step_ms": round(step_ms, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "tflops": round(step_tf, 2),
        "frac_of_peak": round(step_tf / PEAK_BF16_TFLOPS, 4),
        "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "flop_convention": "4*d per visible (query, key) pair of the active blocks forward, backward 2.5x",
    }


def bench_dropout(fa2, workloads, steps, warmup, p=0.1):
    """Dense causal workload (B=4, H=32, N=8192, d=128) with dropout p on the attention weights:
    fa2_fwd_dropout + fa2_bwd_dropout, timed with events; FLOPs as for the dense step."""
    import torch
    w = workloads.WORKLOADS[3]
    B, H, N, d = w.B, w.H, w.N, w.d
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=w.number, with_dout=True)
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "dout"))
    del t
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa2.fa2_bwd_workspace_size(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    seed, offset = 2024, 0

    def fwd():
        fa2.fa2_fwd_dropout(q, k, v, out, lse, B, H, N, d, w.scale, 1, -1, -1, None, p, seed, offset, sp)

    def bwd():
        fa2.fa2_bwd_dropout(q, k, v, out, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, w.scale, 1, -1, -1, None, p,
                            seed, offset, sp)

    ms = timed([("fwd", fwd), ("bwd", bwd)], steps, warmup, stream)
    f_fwd, f_bwd = flops(B, H, N, d, True)
    fwd_tf = f_fwd / (ms["fwd"] * 1e-3) / 1e12
    bwd_tf = f_bwd / (ms["bwd"] * 1e-3) / 1e12
    step_ms = ms["fwd"] + ms["bwd"]
    step_tf = (f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12
    return {
        "workload": f"bf16 causal attention fwd+bwd with dropout p={p}, B={B} H={H} N={N} d={d}",
        "fwd_ms": round(ms["fwd"], 4),
        "bwd_ms": round(ms["bwd"], 4),
        "step_ms": round(step_ms, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "tflops": round(step_tf, 2),
        "frac_of_peak": round(step_tf / PEAK_BF16_TFLOPS, 4),
        "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "flop_convention": "as the dense step: forward 4*B*H*N^2*d/2, backward 2.5x",
    }


def visible_pairs(B, H, N, causal, wl, wr):
    """Number of visible (query, key) pairs under the causal / window rule."""
    import numpy as np
    i = np.arange(N, dtype=np.float64)
    lo = np.zeros(N) if wl < 0 else np.maximum(i - wl, 0)
    hi = i if causal else (np.full(N, N - 1.0) if wr < 0 else np.minimum(i + wr, N - 1))
    return float(B * H * (hi - lo + 1).sum())


def bench_other_workloads(fa2, workloads, steps, warmup):
    """fa2_fwd and fa2_bwd on the dense workloads other than the headline one. TFLOP/s in the
    workload convention (4*B*H*N^2*d, halved for causal; backward 2.5x) and algorithmic (4*d FLOP per
    visible pair forward, 10*d backward). The d=64 workload (134 MB of inputs) fits the 256 MB
    Infinity Cache, so it is also timed with a 512 MB write between launches."""
    import torch
    res = {}
    # The tiny float32 workload (B=1, H=2, N=128, d=64): latency only (two workgroups).
    w1 = workloads.WORKLOADS[1]
    t1 = workloads.make_inputs(w1.B, w1.H, w1.N, w1.d, "f32", seed=w1.number)
    q1, k1, v1 = (t1[n].cuda() for n in ("q", "k", "v"))
    o1 = torch.empty_like(q1)
    l1 = torch.empty((w1.B, w1.H, w1.N), dtype=torch.float32, device="cuda")
    s1 = torch.cuda.current_stream()
    st1 = timed_stats([("fwd", lambda: fa2.fa2_fwd_f32(q1, k1, v1, o1, l1, w1.B, w1.H, w1.N, w1.d, w1.scale,
                                                       int(w1.causal), -1, -1, None, s1.cuda_stream))],
                      steps, warmup, s1)
    res[w1.name] = {"workload": w1.describe(), "fwd_us_median": round(1e3 * st1["fwd"]["median_ms"], 2),
                    "fwd_us_min": round(1e3 * st1["fwd"]["min_ms"], 2)}
    del q1, k1, v1, o1, l1
    for num in (2, 4, 5):
        w = workloads.WORKLOADS[num]
        B, H, N, d = w.B, w.H, w.N, w.d
        t = workloads.make_inputs(B, H, N, d, "bf16", seed=w.number, with_dout=True)
        q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "dout"))
        del t
        out = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = fa2.fa2_bwd_workspace_size(B, H, N, d)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        sl = workloads.alibi_slopes(H).cuda() if w.alibi else None
        c, (wl, wr) = int(w.causal), w.window
        stream = torch.cuda.current_stream()
        sp = stream.cuda_stream

        def fwd():
            fa2.fa2_fwd(q, k, v, out, lse, B, H, N, d, w.scale, c, wl, wr, sl, sp)

        def bwd():
            fa2.fa2_bwd(q, k, v, out, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, w.scale, c, wl, wr, sl, 1, sp)

        st = timed_stats([("fwd", fwd), ("bwd", bwd)], steps, warmup, stream)
        ms = {k: v["avg_ms"] for k, v in st.items()}
        nominal = 4.0 * B * H * N * N * d * (0.5 if w.causal else 1.0)
        pairs = visible_pairs(B, H, N, w.causal, wl, wr)
        fwd_alg = 4.0 * d * pairs / (ms["fwd"] * 1e-3) / 1e12
        rec = {
            "workload": w.describe(),
            "fwd_ms": round(ms["fwd"], 4),
            "bwd_ms": round(ms["bwd"], 4),
            "fwd_ms_median": round(st["fwd"]["median_ms"], 4),
            "fwd_ms_min": round(st["fwd"]["min_ms"], 4),
            "bwd_ms_median": round(st["bwd"]["median_ms"], 4),
            "bwd_ms_min": round(st["bwd"]["min_ms"], 4),
            "fwd_tflops": round(nominal / (ms["fwd"] * 1e-3) / 1e12, 2),
            "bwd_tflops": round(2.5 * nominal / (ms["bwd"] * 1e-3) / 1e12, 2),
            "fwd_tflops_algorithmic": round(fwd_alg, 2),
            "bwd_tflops_algorithmic": round(10.0 * d * pairs / (ms["bwd"] * 1e-3) / 1e12, 2),
            "fwd_frac_of_peak_algorithmic": round(fwd_alg / PEAK_BF16_TFLOPS, 4),
        }
        if num == 2:
            flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
            ms_f = timed([("flush", lambda: flush.fill_(1)), ("fwd", fwd)], steps, warmup, stream)
            rec["fwd_ms_cold_cache"] = round(ms_f["fwd"], 4)
            rec["fwd_tflops_cold_cache"] = round(nominal / (ms_f["fwd"] * 1e-3) / 1e12, 2)
            del flush
        res[w.name] = rec
        del q, k, v, do, out, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return res


def recorded_traffic(call):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (profiles/hbm_traffic.json), reported only if
    the kernel sources still hash to the values the counters were taken with."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    ent = rec.get("kernels", {}).get(call)
    if not ent:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return ent["hbm_bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other dense workloads (d=64 non-causal, N=4096 causal, N=16384 window + ALiBi)")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed variable-length measurement")
    ap.add_argument("--varlen-only", action="store_true",
                    help="only time the packed variable-length workload (prints its object as the JSON line)")
    ap.add_argument("--no-sparse", action="store_true", help="skip the block-sparse measurement")
    ap.add_argument("--sparse-only", action="store_true",
                    help="only time the block-sparse workload (prints its object as the JSON line)")
    ap.add_argument("--no-dropout", action="store_true", help="skip the dropout measurement")
    ap.add_argument("--dropout-only", action="store_true",
                    help="only time the dropout workload (prints its object as the JSON line)")
    ap.add_argument("--other-workloads", action="store_true",
                    help="only time the other dense workloads (prints their objects as the JSON line)")
    ap.add_argument("--atomic-dq", action="store_true",
                    help="time the float-atomic dQ variant of the backward instead of the default passes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 launches), used to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters against a known byte count")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path shards by "
              f"(batch, head) with no exchange, so one GPU's share is what this measures)", file=sys.stderr)
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
    if args.varlen_only:
        print(json.dumps({"varlen": bench_varlen(fa2, workloads, args.steps, args.warmup)}), flush=True)
        return
    if args.sparse_only:
        print(json.dumps({"blocksparse": bench_blocksparse(fa2, workloads, args.steps, args.warmup)}), flush=True)
        return
    if args.other_workloads:
        print(json.dumps({"other_workloads": bench_other_workloads(fa2, workloads, args.steps, args.warmup)}),
              flush=True)
        return
    if args.dropout_only:
        print(json.dumps({"dropout": bench_dropout(fa2, workloads, args.steps, args.warmup)}), flush=True)
        return
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

    def fwd():
        fa2.fa2_fwd(q, k, v, out, lse, B, H, N, d, scale, 1, -1, -1, None, sp)

    # The backward as its two passes (exactly what fa2_bwd runs by default: the dQ pass,
    # which also forms D and the per-row values, then the dK/dV pass), so each kernel's
    # duration is measured with its own events.
    def dkdv():
        fa2.fa2_bwd_dkdv(q, k, v, lse, do, dk, dv, ws, ws_bytes, B, H, N, d, scale, 1, -1, -1, None, sp)

    def dqp():
        fa2.fa2_bwd_dq_stats(q, k, v, out, lse, do, dq, ws, ws_bytes, B, H, N, d, scale, 1, -1, -1, None, sp)

    def bwd_atomic():
        fa2.fa2_bwd(q, k, v, out, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, scale, 1, -1, -1, None, 0, sp)

    phases = [("fwd", fwd), ("bwd_dq", dqp), ("bwd_dkdv", dkdv)]
    if args.atomic_dq:
        os.environ["FA2_BWD_ATOMIC_DQ"] = "1"
        phases = [("fwd", fwd), ("bwd_atomic", bwd_atomic)]

    for _ in range(args.warmup):
        for _, fn in phases:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        for n, (_, fn) in enumerate(phases):
            fn()
            ev[i][n + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / K
    ph_stats = {name: phase_stats([e[n].elapsed_time(e[n + 1]) for e in ev]) for n, (name, _) in enumerate(phases)}
    ph_ms = {name: st["avg_ms"] for name, st in ph_stats.items()}
    f_fwd, f_bwd = flops(B, H, N, d, True)
    pairs = B * H * N * (N + 1) / 2  # visible (query, key) pairs, causal
    fwd_avg = ph_ms["fwd"]
    bwd_avg = sum(v for kk, v in ph_ms.items() if kk != "fwd")
    fwd_tf = f_fwd / (fwd_avg * 1e-3) / 1e12
    bwd_tf = f_bwd / (bwd_avg * 1e-3) / 1e12
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    # Per-kernel rooflines. Executed MFMA FLOPs per launch: forward 4*d per visible
    # pair (S, P V); dK/dV pass 8*d (S, dP, dV, dK); dQ pass 6*d (S, dP, dQ).
    kinfo = {
        "fwd": ("fwd_bf16_kernel", 4 * d * pairs),
        "bwd_dkdv": ("bwd_main_kernel (dK, dV)", 8 * d * pairs),
        "bwd_dq": ("bwd_dq_det_kernel (dQ, with D)", 6 * d * pairs),
    }
    kernels = {}
    for name, ms in ph_ms.items():
        ent = {k: round(v, 4) for k, v in ph_stats[name].items()}
        if name in kinfo:
            kn, fl = kinfo[name]
            ach = fl / (ms * 1e-3) / 1e12
            ach_med = fl / (ph_stats[name]["median_ms"] * 1e-3) / 1e12
            ent.update({"kernel": kn, "bound": "mfma", "flop_per_launch": fl, "achieved": round(ach, 2),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                        "frac_median": round(ach_med / PEAK_BF16_TFLOPS, 4)})
        kernels[name] = ent
    dom = max((n for n in kernels if "frac" in kernels[n]), key=lambda n: kernels[n]["avg_ms"])
    dk_ = kernels[dom]
    traffic = recorded_traffic(dom)
    # Compulsory HBM bytes per launch: each tensor of B*N*H*d bf16 values read or
    # written once, plus the per-row fp32 statistics.
    tb, sb = B * N * H * d * 2, B * H * N * 4
    compulsory = {"fwd": 3 * tb + (tb + sb), "bwd_dq": (5 * tb + sb) + (tb + 2 * sb),
                  "bwd_dkdv": (4 * tb + 2 * sb) + 2 * tb}[dom]
    roofline = {"bound": "mfma", "achieved": dk_["achieved"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": dk_["frac"], "traffic": traffic, "kernel": dk_["kernel"], "call": dom,
                "compulsory_bytes": compulsory,
                "traffic_over_compulsory": None if traffic is None else round(traffic / compulsory, 3)}

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
                   "parallelism": "none (1 GPU)",
                   "bwd_dq": "float atomics" if args.atomic_dq else "separate pass (no atomics)"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_other:
        rec["other_workloads"] = bench_other_workloads(fa2, workloads, args.steps, args.warmup)
    if not args.no_varlen:
        rec["varlen"] = bench_varlen(fa2, workloads, args.steps, args.warmup)
    if not args.no_sparse:
        rec["blocksparse"] = bench_blocksparse(fa2, workloads, args.steps, args.warmup)
        rec["blocksparse"]["speedup_vs_dense_step"] = round(ms_step / rec["blocksparse"]["step_ms"], 3)
    if not args.no_dropout:
        rec["dropout"] = bench_dropout(fa2, workloads, args.steps, args.warmup)
        rec["dropout"]["slowdown_vs_dense_step"] = round(rec["dropout"]["step_ms"] / ms_step, 3)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
