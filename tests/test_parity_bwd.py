"""Backward parity: HIP gradients (through the C ABI) against the fp64 oracle.

The forward's own O and LSE (from the HIP path) feed the HIP backward, as in
use; the oracle recomputes everything from q, k, v, dout by the definition.
Metric: max |error| / max |reference| per tensor <= 5e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import TOL_GRAD_REL, edge_rows, gpu_inputs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu

MASKS = {
    "full": (False, (-1, -1), False),
    "causal": (True, (-1, -1), False),
    "window_37_5": (False, (37, 5), False),
    "causal_window_70": (True, (70, 0), False),
    "causal_window_alibi": (True, (100, 0), True),
    "alibi_noncausal": (False, (-1, -1), True),
    "window_0_0": (False, (0, 0), False),
}


def run_fwd_bwd(fa2, dev, slopes, scale, causal, window, deterministic=False):
    """deterministic: False = library default, True = deterministic flag, "atomic" =
    the float-atomic dQ variant (FA2_BWD_ATOMIC_DQ=1 with deterministic = 0)."""
    import os
    atomic = deterministic == "atomic"
    if atomic:
        os.environ["FA2_BWD_ATOMIC_DQ"] = "1"
        deterministic = False
    sl = None if slopes is None else slopes.cuda()
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, causal, window, sl)
    try:
        dq, dk, dv = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale, causal, window,
                                        sl, deterministic)
        torch.cuda.synchronize()
    finally:
        if atomic:
            del os.environ["FA2_BWD_ATOMIC_DQ"]
    return dq, dk, dv


def check_small(fa2, B, H, N, d, causal, window, alibi, deterministic, seed):
    cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=seed, with_dout=True, alibi=alibi)
    dq, dk, dv = run_fwd_bwd(fa2, dev, slopes, scale_of(d), causal, window, deterministic)
    gq, gk, gv = oracle.attention_backward(cpu["q"], cpu["k"], cpu["v"], cpu["dout"], scale_of(d), causal, window,
                                           None if slopes is None else slopes.numpy())
    errs = [rel_to_max(to_np(x), r) for x, r in ((dq, gq), (dk, gk), (dv, gv))]
    say(f"  rel-to-max err dq={errs[0]:.3e} dk={errs[1]:.3e} dv={errs[2]:.3e}")
    assert max(errs) <= TOL_GRAD_REL, errs
    return dq, dk, dv


@pytest.mark.parametrize("deterministic", [False, True, "atomic"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", sorted(MASKS))
def test_small_bf16_gradients(gpu_lib, d, mask, deterministic):
    causal, window, alibi = MASKS[mask]
    say(f"bwd bf16 small d={d} mask={mask} det={deterministic}")
    check_small(gpu_lib, 2, 3, 301, d, causal, window, alibi, deterministic, seed=31 + d)


@pytest.mark.parametrize("N", [1, 17, 128, 129, 200])
def test_edge_lengths(gpu_lib, N):
    say(f"bwd bf16 edge N={N}")
    check_small(gpu_lib, 1, 2, N, 128, True, (-1, -1), False, False, seed=N + 100)


@pytest.mark.parametrize("deterministic", [False, True, "atomic"])
def test_self_only_window_has_zero_dq_dk(gpu_lib, deterministic):
    """window (0, 0): each query sees only itself, P = 1, D = dP, so dS = 0: dQ = dK = 0 and dV = dO."""
    cpu, dev, _ = gpu_inputs(1, 2, 190, 128, "bf16", seed=43, with_dout=True)
    dq, dk, dv = run_fwd_bwd(gpu_lib, dev, None, scale_of(128), False, (0, 0), deterministic)
    assert float(dq.abs().max()) < 1e-4 and float(dk.abs().max()) < 1e-4
    assert torch.equal(dv.cpu(), cpu["dout"])


@pytest.mark.parametrize("deterministic", [False, True])
def test_bitwise_repeatable(gpu_lib, deterministic):
    cpu, dev, slopes = gpu_inputs(1, 4, 700, 128, "bf16", seed=41, with_dout=True, alibi=True)
    a = run_fwd_bwd(gpu_lib, dev, slopes, scale_of(128), True, (200, 0), deterministic=deterministic)
    b = run_fwd_bwd(gpu_lib, dev, slopes, scale_of(128), True, (200, 0), deterministic=deterministic)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dv_columns_sum_to_dout_columns(gpu_lib):
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i for every head (a property at any size)."""
    cpu, dev, _ = gpu_inputs(2, 2, 513, 64, "bf16", seed=42, with_dout=True)
    _, _, dv = run_fwd_bwd(gpu_lib, dev, None, scale_of(64), True, (-1, -1))
    lhs = dv.double().sum(1).cpu().numpy()
    rhs = cpu["dout"].double().sum(1).numpy()
    assert np.max(np.abs(lhs - rhs)) / np.max(np.abs(rhs)) < 2e-2


@pytest.mark.parametrize("deterministic", [False, "atomic"])
@pytest.mark.parametrize("number", [2, 3, 4, 5])
def test_full_size_workload_sampled_rows(gpu_lib, number, deterministic):
    w = workloads.WORKLOADS[number]
    say(f"bwd full-size {w.describe()} det={deterministic}")
    t = workloads.workload_inputs(w, with_dout=True)
    dev = {k: t[k].cuda() for k in ("q", "k", "v", "dout")}
    dq, dk, dv = run_fwd_bwd(gpu_lib, dev, t["alibi_slopes"], w.scale, w.causal, w.window, deterministic)
    qrows = workloads.sample_query_rows(w.B, w.H, w.N, 256, seed=1000 + number)
    qrows = np.concatenate([qrows, edge_rows(w.B, w.H, w.N, extra=(1, 128, w.window[0]))])
    krows = workloads.sample_key_rows(w.B, w.H, w.N, 256, max_heads=2, seed=1000 + number)
    sl = None if t["alibi_slopes"] is None else t["alibi_slopes"].numpy()
    gq, gk, gv = oracle.attention_backward_sampled(t["q"], t["k"], t["v"], t["dout"], qrows, krows, w.scale,
                                                   w.causal, w.window, sl)
    dq_np, dk_np, dv_np = (x.float().cpu().numpy() for x in (dq, dk, dv))
    e_q = rel_to_max(dq_np[qrows[:, 0], qrows[:, 2], qrows[:, 1]], gq)
    e_k = rel_to_max(dk_np[krows[:, 0], krows[:, 2], krows[:, 1]], gk)
    e_v = rel_to_max(dv_np[krows[:, 0], krows[:, 2], krows[:, 1]], gv)
    say(f"  rel-to-max err dq={e_q:.3e} dk={e_k:.3e} dv={e_v:.3e}")
    assert max(e_q, e_k, e_v) <= TOL_GRAD_REL
    for x in (dq_np, dk_np, dv_np):
        assert np.isfinite(x).all()


@pytest.mark.parametrize("d", [64, 128])
def test_pass_entry_points_match_fa2_bwd_on_two_streams(gpu_lib, d):
    """fa2_bwd_prep, then fa2_bwd_dkdv and fa2_bwd_dq on two streams, equal fa2_bwd bitwise."""
    B, H, N = 2, 3, 450
    cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=44, with_dout=True, alibi=True)
    sl = slopes.cuda()
    scale = scale_of(d)
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, True, (200, 0), sl)
    ref = gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale, True, (200, 0), sl)
    ws_bytes = 2 * ((B * H * N * 4 + 255) // 256 * 256)  # -D and -LSE / scale per row
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    gpu_lib.fa2_bwd_prep(out, dev["dout"], lse, ws, ws_bytes, B, H, N, d, scale, s0.cuda_stream)
    ev = torch.cuda.Event()
    ev.record(s0)
    s1.wait_event(ev)
    gpu_lib.fa2_bwd_dkdv(dev["q"], dev["k"], dev["v"], lse, dev["dout"], dk, dv, ws, ws_bytes, B, H, N, d, scale,
                         1, 200, 0, sl, s0.cuda_stream)
    gpu_lib.fa2_bwd_dq(dev["q"], dev["k"], dev["v"], lse, dev["dout"], dq, ws, ws_bytes, B, H, N, d, scale, 1,
                       200, 0, sl, s1.cuda_stream)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_fused_dq_pass_writes_the_prep_values_and_matches_fa2_bwd(gpu_lib, d):
    """fa2_bwd_dq_stats writes the workspace fa2_bwd_prep writes, bit for bit, and
    fa2_bwd_dq_stats then fa2_bwd_dkdv equal fa2_bwd bitwise."""
    B, H, N = 2, 3, 450
    cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=46, with_dout=True, alibi=True)
    sl = slopes.cuda()
    scale = scale_of(d)
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, True, (200, 0), sl)
    ref = gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale, True, (200, 0), sl)
    ws_bytes = 2 * ((B * H * N * 4 + 255) // 256 * 256)
    ws_prep = torch.full((ws_bytes,), 0x7F, dtype=torch.uint8, device="cuda")
    ws = torch.full((ws_bytes,), 0x7F, dtype=torch.uint8, device="cuda")
    gpu_lib.fa2_bwd_prep(out, dev["dout"], lse, ws_prep, ws_bytes, B, H, N, d, scale, None)
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    gpu_lib.fa2_bwd_dq_stats(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], dq, ws, ws_bytes, B, H, N, d,
                             scale, 1, 200, 0, sl, None)
    gpu_lib.fa2_bwd_dkdv(dev["q"], dev["k"], dev["v"], lse, dev["dout"], dk, dv, ws, ws_bytes, B, H, N, d, scale,
                         1, 200, 0, sl, None)
    torch.cuda.synchronize()
    assert torch.equal(ws, ws_prep)
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_prep_pass_writes_minus_d_and_minus_lse_over_scale(gpu_lib, d):
    """fa2_bwd_prep's workspace: -D per row (D = rowsum(dO * O), fp64 from the given O
    and dO) at offset 0, then -LSE / scale per row, each array rounded up to 256 bytes."""
    B, H, N = 2, 3, 77
    cpu, dev, _ = gpu_inputs(B, H, N, d, "bf16", seed=45, with_dout=True)
    scale = scale_of(d)
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, True, (-1, -1), None)
    rows = B * H * N
    part = (rows * 4 + 255) // 256 * 256
    ws = torch.full((2 * part,), 0xFF, dtype=torch.uint8, device="cuda")
    gpu_lib.fa2_bwd_prep(out, dev["dout"], lse, ws, 2 * part, B, H, N, d, scale, None)
    torch.cuda.synchronize()
    nd = ws[:rows * 4].view(torch.float32).cpu().numpy().reshape(B, H, N)
    si = ws[part:part + rows * 4].view(torch.float32).cpu().numpy().reshape(B, H, N)
    o = to_np(out).astype(np.float64)
    do = cpu["dout"].double().numpy()
    d_ref = np.einsum("bnhd,bnhd->bhn", o, do)
    assert np.max(np.abs(nd + d_ref)) <= 1e-4 * max(1.0, np.max(np.abs(d_ref)))
    lse_np = lse.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(si, -lse_np / scale, rtol=1e-6, atol=1e-6)


def test_backward_window_beyond_int_range_is_unbounded(gpu_lib):
    """window_size = (2^31 - 1, 2^31 - 1) in the backward: bit for bit the gradients of (-1, -1)."""
    big = 2**31 - 1
    _, dev, _ = gpu_inputs(1, 2, 300, 128, "bf16", seed=43, with_dout=True)
    for causal in (False, True):
        a = run_fwd_bwd(gpu_lib, dev, None, scale_of(128), causal, (big, big), True)
        b = run_fwd_bwd(gpu_lib, dev, None, scale_of(128), causal, (-1, -1), True)
        assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("bad", ["bf16", "transposed", "short", "cpu", "workspace_cpu"])
def test_backward_rejects_a_malformed_lse(gpu_lib, bad):
    """The wrappers check lse (float32, contiguous, [B, H, N], on the tensors' GPU) and the
    workspace's device before anything is launched."""
    B, H, N, d = 1, 2, 64, 64
    _, dev, _ = gpu_inputs(B, H, N, d, "bf16", seed=44, with_dout=True)
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale_of(d))
    ws = None
    if bad == "bf16":
        lse = lse.to(torch.bfloat16)
    elif bad == "transposed":
        lse = lse.transpose(1, 2).contiguous()  # [B, N, H]
    elif bad == "short":
        lse = lse[:, :, : N - 1].contiguous()
    elif bad == "cpu":
        lse = lse.cpu()
    else:
        ws = torch.empty(1 << 16, dtype=torch.uint8)
    with pytest.raises(gpu_lib.FA2Error):
        gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale_of(d), workspace=ws)
    packed = {k: v.reshape(B * N, H, d) for k, v in dev.items()}
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    o2, l2 = gpu_lib.flash_attn_varlen_fwd(packed["q"], packed["k"], packed["v"], cu, scale_of(d))
    with pytest.raises(gpu_lib.FA2Error):
        gpu_lib.flash_attn_varlen_bwd(packed["dout"], packed["q"], packed["k"], packed["v"], o2,
                                      l2.reshape(1, H, N), cu, scale_of(d))
