"""Forward parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element on every output; they span
several 64-key tiles and 128-row query blocks and end in a ragged tail. The
full-size workloads are compared on 256 seeded query rows plus fixed edge rows,
in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import (TOL_LSE, TOL_O_BF16, TOL_O_F32, edge_rows, gather_lse, gather_rows,
                          gpu_inputs, max_abs, oracle_forward_rows, say, scale_of, to_np)

pytestmark = pytest.mark.gpu

MASKS = {
    "full": (False, (-1, -1), False),
    "causal": (True, (-1, -1), False),
    "window_37_5": (False, (37, 5), False),
    "window_0_0": (False, (0, 0), False),
    "causal_window_70": (True, (70, 0), False),
    "causal_window_alibi": (True, (100, 0), True),
    "alibi_noncausal": (False, (-1, -1), True),
    "window_left_only": (False, (50, -1), False),
}


def run_fwd(fa2, dev, slopes, scale, causal, window):
    sl = None if slopes is None else slopes.cuda()
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, causal, window, sl)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", sorted(MASKS))
def test_small_bf16_all_outputs(gpu_lib, d, mask):
    causal, window, alibi = MASKS[mask]
    B, H, N = 2, 3, 301  # 3 query blocks of 128 rows, 5 key tiles of 64, ragged tail
    say(f"fwd bf16 small d={d} mask={mask} B={B} H={H} N={N}")
    cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=11 + d, alibi=alibi)
    out, lse = run_fwd(gpu_lib, dev, slopes, scale_of(d), causal, window)
    o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], scale_of(d), causal, window,
                                              None if slopes is None else slopes.numpy())
    eo, el = max_abs(to_np(out), o_ref), max_abs(to_np(lse), lse_ref)
    say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 128, 129, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths(gpu_lib, N, causal):
    say(f"fwd bf16 edge N={N} causal={causal}")
    cpu, dev, _ = gpu_inputs(1, 2, N, 128, "bf16", seed=N)
    out, lse = run_fwd(gpu_lib, dev, None, scale_of(128), causal, (-1, -1))
    o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], scale_of(128), causal)
    assert max_abs(to_np(out), o_ref) <= TOL_O_BF16
    assert max_abs(to_np(lse), lse_ref) <= TOL_LSE
    if causal:
        # causal row 0 is exactly V[0] and its LSE is scale * q0.k0
        assert torch.equal(out[:, 0].cpu(), cpu["v"][:, 0])


def test_single_key_returns_v(gpu_lib):
    cpu, dev, _ = gpu_inputs(3, 4, 1, 64, "bf16", seed=5)
    out, lse = run_fwd(gpu_lib, dev, None, 0.3, False, (-1, -1))
    assert torch.equal(out.cpu(), cpu["v"])
    ref = 0.3 * torch.einsum("bnhd,bnhd->bhn", cpu["q"].double(), cpu["k"].double())
    assert max_abs(to_np(lse), ref.numpy()) <= TOL_LSE


def test_constant_v(gpu_lib):
    cpu, dev, _ = gpu_inputs(1, 2, 257, 128, "bf16", seed=6)
    row = torch.linspace(-2, 2, 128).to(torch.bfloat16)
    dev["v"] = row.expand(1, 257, 2, 128).contiguous().cuda()
    out, _ = run_fwd(gpu_lib, dev, None, scale_of(128), True, (40, 0))
    assert max_abs(to_np(out), row.float().expand(1, 257, 2, 128).numpy()) <= 1e-2


def test_tiny_fp32_workload_full_check(gpu_lib):
    w = workloads.WORKLOADS[1]
    say(f"fwd {w.describe()}")
    t = workloads.workload_inputs(w)
    out, lse = run_fwd(gpu_lib, {k: t[k].cuda() for k in ("q", "k", "v")}, None, w.scale, w.causal, w.window)
    o_ref, lse_ref = oracle.attention_forward(t["q"], t["k"], t["v"], w.scale, w.causal, w.window)
    eo, el = max_abs(to_np(out), o_ref), max_abs(to_np(lse), lse_ref)
    say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O_F32 and el <= TOL_O_F32


@pytest.mark.parametrize("mask", ["full", "causal", "causal_window_alibi", "window_37_5"])
def test_fp32_small_masks(gpu_lib, mask):
    causal, window, alibi = MASKS[mask]
    cpu, dev, slopes = gpu_inputs(2, 2, 150, 64, "f32", seed=9, alibi=alibi)
    out, lse = run_fwd(gpu_lib, dev, slopes, 0.125, causal, window)
    o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], 0.125, causal, window,
                                              None if slopes is None else slopes.numpy())
    assert max_abs(to_np(out), o_ref) <= TOL_O_F32
    assert max_abs(to_np(lse), lse_ref) <= TOL_O_F32


@pytest.mark.parametrize("mask", sorted(MASKS))
def test_fp32_d128_all_outputs(gpu_lib, mask):
    """The float32-storage forward at d = 128 (the largest register footprint of the
    float32 kernel) against the oracle, every O and LSE element, within the float32
    tolerance; shapes span several key tiles and query blocks and end in a ragged tail."""
    causal, window, alibi = MASKS[mask]
    B, H, N = 1, 3, 291
    say(f"fwd f32 d=128 mask={mask} B={B} H={H} N={N}")
    cpu, dev, slopes = gpu_inputs(B, H, N, 128, "f32", seed=31, alibi=alibi)
    out, lse = run_fwd(gpu_lib, dev, slopes, scale_of(128), causal, window)
    o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], scale_of(128), causal, window,
                                              None if slopes is None else slopes.numpy())
    eo, el = max_abs(to_np(out), o_ref), max_abs(to_np(lse), lse_ref)
    say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O_F32 and el <= TOL_O_F32


@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_window_beyond_int_range_is_unbounded(gpu_lib, dtype, d):
    """window_size = (2^31 - 1, 2^31 - 1) reaches every key: the result must be the one of
    (-1, -1), bit for bit (causal and not), and match the oracle's dense result."""
    big = 2**31 - 1
    cpu, dev, _ = gpu_inputs(1, 2, 333, d, dtype, seed=41)
    for causal in (False, True):
        o1, l1 = run_fwd(gpu_lib, dev, None, scale_of(d), causal, (big, big))
        o2, l2 = run_fwd(gpu_lib, dev, None, scale_of(d), causal, (-1, -1))
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], scale_of(d), causal)
        assert max_abs(to_np(o1), o_ref) <= (TOL_O_F32 if dtype == "f32" else TOL_O_BF16)
        assert max_abs(to_np(l1), lse_ref) <= TOL_LSE


@pytest.mark.parametrize("number", [2, 3, 4, 5])
def test_full_size_workload_sampled_rows(gpu_lib, number):
    w = workloads.WORKLOADS[number]
    say(f"fwd full-size {w.describe()}")
    t = workloads.workload_inputs(w, with_dout=False)
    dev = {k: t[k].cuda() for k in ("q", "k", "v")}
    out, lse = run_fwd(gpu_lib, dev, t["alibi_slopes"], w.scale, w.causal, w.window)
    rows = workloads.sample_query_rows(w.B, w.H, w.N, 256, seed=1000 + number)
    rows = np.concatenate([rows, edge_rows(w.B, w.H, w.N, extra=(1, 127, 128, w.window[0], w.window[0] + 1))])
    o_ref, lse_ref = oracle_forward_rows(t, rows, w.scale, w.causal, w.window, t["alibi_slopes"])
    o_np = out.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    eo = max_abs(gather_rows(o_np, rows), o_ref)
    el = max_abs(gather_lse(lse_np, rows), lse_ref)
    say(f"  rows={len(rows)} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()


def test_forward_is_bitwise_repeatable(gpu_lib):
    cpu, dev, slopes = gpu_inputs(2, 4, 1000, 128, "bf16", seed=21, alibi=True)
    o1, l1 = run_fwd(gpu_lib, dev, slopes, scale_of(128), True, (300, 0))
    o2, l2 = run_fwd(gpu_lib, dev, slopes, scale_of(128), True, (300, 0))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_explicit_stream(gpu_lib):
    cpu, dev, _ = gpu_inputs(1, 2, 130, 64, "bf16", seed=3)
    s = torch.cuda.Stream()
    out = torch.empty_like(dev["q"])
    lse = torch.empty((1, 2, 130), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        gpu_lib.fa2_fwd(dev["q"], dev["k"], dev["v"], out, lse, 1, 2, 130, 64, 0.125, 0, -1, -1, None,
                        s.cuda_stream)
    s.synchronize()
    o_ref, _ = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], 0.125)
    assert max_abs(to_np(out), o_ref) <= TOL_O_BF16


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits): 2^(floor(log2|x|) - 7)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("d,causal,window,alibi", [(128, True, (-1, -1), False), (64, False, (40, 9), True),
                                                     (128, False, (-1, -1), False)])
def test_error_within_the_bf16_rounding_bound(gpu_lib, d, causal, window, alibi):
    """Every O element against a bound derived from the arithmetic rather than a flat
    tolerance: the kernel rounds each weight P_ij to bf16 before P.V (relative error at
    most 2^-8) and rounds O to bf16 once (half a bf16 ulp), so
      |O_gpu - O| <= ulp(O) / 2 + 2^-8 * sum_j P_ij |v_j| + 1e-5
    (fp32 accumulation and the exponential add far less than the slack). The
    distribution of the error against |O| is printed."""
    B, H, N = 1, 2, 700
    cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=77 + d, alibi=alibi)
    sc = scale_of(d)
    out, lse = run_fwd(gpu_lib, dev, slopes, sc, causal, window)
    q, k, v = (cpu[n].double().numpy() for n in ("q", "k", "v"))
    o_gpu = to_np(out).astype(np.float64)
    sl = None if slopes is None else slopes.numpy()
    worst = 0.0
    hist = np.zeros(4)
    for h in range(H):
        s = oracle.logits(q[0, :, h, :], k[0, :, h, :], np.arange(N), sc, causal, window[0], window[1],
                          None if sl is None else float(sl[h]))
        pm, _ = oracle.softmax_rows(s)
        o_ref = pm @ v[0, :, h, :]
        err = np.abs(o_gpu[0, :, h, :] - o_ref)
        bound = 0.5 * np.maximum(bf16_ulp(o_ref), bf16_ulp(o_gpu[0, :, h, :])) + 2.0 ** -8 * (pm @ np.abs(v[0, :, h, :])) + 1e-5
        worst = max(worst, float(np.max(err / bound)))
        mag = np.abs(o_ref)
        for i, (lo, hi) in enumerate([(0, 0.25), (0.25, 1), (1, 4), (4, np.inf)]):
            sel = (mag >= lo) & (mag < hi)
            if sel.any():
                hist[i] = max(hist[i], float(err[sel].max()))
    say(f"  max err by |O| in [0,.25) [.25,1) [1,4) [4,inf): {hist[0]:.2e} {hist[1]:.2e} {hist[2]:.2e} {hist[3]:.2e}; "
        f"worst err/bound {worst:.3f}")
    assert worst <= 1.0
    assert np.max(hist) <= TOL_O_BF16
