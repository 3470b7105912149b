"""Numerically awkward inputs for the online softmax, HIP path (through the C ABI)
against the fp64 oracle, every output element checked:

* large logits: q and k scaled by 8, so the scaled scores span hundreds of units and
  each row's softmax is dominated by a few keys;
* a running maximum that grows on every key tile: steep ALiBi slopes make each row's
  scores rise towards the diagonal fast enough (14-23 log2 units per 32 keys) that
  the forward's deferred rescale fires on every tile of every row;
* uniform rows: q = 0, so every visible key has the same score; O is the mean of the
  visible values and LSE = ln(number of visible keys), closed forms checked as well.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import TOL_GRAD_REL, TOL_LSE, TOL_O_BF16, max_abs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu


def run_and_check(fa2, t, d, causal, window, tag):
    dev = {k: v.cuda() for k, v in t.items()}
    sc = scale_of(d)
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], sc, causal, window, None)
    dq, dk, dv = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, sc, causal, window, None,
                                    True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(t["q"], t["k"], t["v"], sc, causal, window)
    g_ref = oracle.attention_backward(t["q"], t["k"], t["v"], t["dout"], sc, causal, window)
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  {tag}: O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL
    return out, lse


def bf16(x):
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_large_logits(gpu_lib, d, causal):
    B, H, N = 1, 2, 333
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=300 + d, with_dout=True)
    t["q"] = bf16(t["q"].float() * 8)
    t["k"] = bf16(t["k"].float() * 8)
    run_and_check(gpu_lib, t, d, causal, (-1, -1), f"large logits d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_running_max_grows_on_every_tile(gpu_lib, d):
    """Steep ALiBi slopes (0.3 and 0.5 per position) under a causal mask: a row's scores
    rise by 32 * slope * log2(e) = 14-23 log2 units per 32-key tile towards the
    diagonal, so the forward's deferred rescale (threshold 8) fires on every tile."""
    B, H, N = 1, 2, 512
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=310 + d, with_dout=True)
    slopes = torch.tensor([0.3, 0.5], dtype=torch.float32)
    dev = {k: v.cuda() for k, v in t.items()}
    sc = scale_of(d)
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], sc, True, (-1, -1), slopes.cuda())
    dq, dk, dv = gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, sc, True, (-1, -1),
                                        slopes.cuda(), True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(t["q"], t["k"], t["v"], sc, True, (-1, -1), slopes.numpy())
    g_ref = oracle.attention_backward(t["q"], t["k"], t["v"], t["dout"], sc, True, (-1, -1), slopes.numpy())
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  rising scores d={d}: O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [(-1, -1), (40, 0), (25, 7)])
def test_uniform_rows_closed_form(gpu_lib, d, window):
    B, H, N = 1, 2, 300
    causal = window == (40, 0)
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=320 + d, with_dout=True)
    t["q"] = torch.zeros_like(t["q"])
    out, lse = run_and_check(gpu_lib, t, d, causal, window, f"q = 0 d={d} window={window}")
    # closed forms: key j visible to row i iff i - wl <= j <= i + wr (causal: wr = 0)
    wl, wr = window
    wr = 0 if causal else wr
    i = np.arange(N)
    lo = np.maximum(0, i - wl) if wl >= 0 else np.zeros(N, dtype=np.int64)
    hi = np.minimum(N - 1, i + wr) if wr >= 0 else np.full(N, N - 1)
    count = hi - lo + 1
    v = t["v"].double().numpy()
    csum = np.concatenate([np.zeros((1,) + v.shape[2:]), np.cumsum(v[0], axis=0)])  # [N + 1, H, d]
    mean = (csum[hi + 1] - csum[lo]) / count[:, None, None]
    assert max_abs(lse.cpu().numpy()[0], np.broadcast_to(np.log(count), (H, N))) <= TOL_LSE
    assert max_abs(to_np(out)[0], mean) <= TOL_O_BF16
