"""Shared helpers for the GPU parity tests: inputs, the oracle side, error metrics."""
import math

import numpy as np
import torch

import oracle
import workloads

# Tolerances (stated on the workload definitions): forward O max abs error
# <= 1e-5 (float32 storage) / 2e-2 (bf16 storage); LSE max abs error <= 1e-3;
# gradients: max |error| / max |reference| <= 5e-2 per tensor.
TOL_O_F32 = 1e-5
TOL_O_BF16 = 2e-2
TOL_LSE = 1e-3
TOL_GRAD_REL = 5e-2


def say(*a):
    print(*a, flush=True)


def gpu_inputs(B, H, N, d, dtype="bf16", seed=0, with_dout=False, alibi=False):
    t = workloads.make_inputs(B, H, N, d, dtype, seed, with_dout)
    dev = {k: v.cuda() for k, v in t.items()}
    slopes = workloads.alibi_slopes(H) if alibi else None
    return t, dev, slopes


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)))) if np.size(a) else 0.0


def rel_to_max(a, ref, floor=1e-3):
    """max |a - ref| / max |ref|. The denominator is floored so that a reference
    that is exactly zero by the mathematics (e.g. dQ and dK when every query sees
    only itself, where dS = 0) turns into an absolute check."""
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    return max_abs(a, ref) / max(denom, floor)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def scale_of(d):
    return 1.0 / math.sqrt(d)


def gather_rows(t_bnhd, rows):
    """t: numpy [B, N, H, d]; rows: [n, 3] (b, h, i) -> [n, d]."""
    return t_bnhd[rows[:, 0], rows[:, 2], rows[:, 1], :]


def gather_lse(lse_bhn, rows):
    return lse_bhn[rows[:, 0], rows[:, 1], rows[:, 2]]


def edge_rows(B, H, N, extra=()):
    """Fixed rows added to a random sample: first and last row of a few heads, and extras."""
    rows = []
    for b, h in {(0, 0), (B - 1, H - 1)}:
        for i in {0, N - 1, *[x for x in extra if 0 <= x < N]}:
            rows.append((b, h, i))
    return np.array(rows, dtype=np.int64)


def oracle_forward_rows(cpu, rows, scale, causal, window, slopes):
    return oracle.attention_forward_rows(cpu["q"], cpu["k"], cpu["v"], rows, scale, causal, window,
                                         None if slopes is None else slopes.numpy())
