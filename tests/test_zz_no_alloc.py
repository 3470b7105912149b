"""The allocation-free backward (fa2_bwd_noalloc) against fa2_bwd, through the C ABI.

fa2_bwd_noalloc keeps its per-row scratch in a device array inside the library
instead of a caller's workspace; it runs the same atomic-free passes, so its
gradients must equal fa2_bwd's (deterministic = 1) bit for bit. Two calls in a
row, the second smaller, check that the array's leftover contents from the first
call do not leak into the second; a call at the array's row limit checks the
largest size it accepts.
"""
import math

import pytest
import torch

import oracle
from parity_utils import TOL_GRAD_REL, gpu_inputs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu


def grads(fa2, dev, slopes, causal, window, noalloc):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["dout"]
    B, N, H, d = q.shape
    sc = scale_of(d)
    sl = None if slopes is None else slopes.cuda()
    out, lse = fa2.flash_attn_fwd(q, k, v, sc, causal, window, sl)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    c = int(bool(causal))
    if noalloc:
        fa2.fa2_bwd_noalloc(q, k, v, out, lse, do, dq, dk, dv, B, H, N, d, sc, c, window[0], window[1], sl)
    else:
        ws_bytes = fa2.fa2_bwd_workspace_size(B, H, N, d)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        fa2.fa2_bwd(q, k, v, out, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, sc, c, window[0], window[1], sl, 1)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_backward_twice(gpu_lib, order):
    cases = [(2, 4, 700, 128, True, (300, 0), True, 51), (1, 2, 130, 64, False, (-1, -1), False, 52)]
    for B, H, N, d, causal, window, alibi, seed in cases:
        say(f"noalloc bwd B={B} H={H} N={N} d={d} causal={causal} window={window} alibi={alibi}")
        cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=seed, with_dout=True, alibi=alibi)
        a = grads(gpu_lib, dev, slopes, causal, window, noalloc=True)
        b = grads(gpu_lib, dev, slopes, causal, window, noalloc=False)
        for name, x, y in zip("qkv", a, b):
            assert torch.equal(x, y), f"d{name} differs from fa2_bwd"
        gq, gk, gv = oracle.attention_backward(cpu["q"], cpu["k"], cpu["v"], cpu["dout"], scale_of(d), causal,
                                               window, None if slopes is None else slopes.numpy())
        errs = [rel_to_max(to_np(x), r) for x, r in zip(a, (gq, gk, gv))]
        say(f"  equal to fa2_bwd; rel-to-max err vs oracle {max(errs):.3e}")
        assert max(errs) <= TOL_GRAD_REL


def test_noalloc_at_its_row_limit(gpu_lib):
    """B * H * N = 2^21 rows, the most the scratch array holds (B=1, H=16, N=131072 would
    exceed the block-sparse limit elsewhere; dense causal has no such limit)."""
    B, H, N, d = 1, 32, 65536, 128
    say(f"noalloc bwd at the limit B={B} H={H} N={N} d={d} causal")
    _, dev, _ = gpu_inputs(B, H, N, d, "bf16", seed=53, with_dout=True)
    a = grads(gpu_lib, dev, None, True, (-1, -1), noalloc=True)
    b = grads(gpu_lib, dev, None, True, (-1, -1), noalloc=False)
    for name, x, y in zip("qkv", a, b):
        assert torch.equal(x, y), f"d{name} differs from fa2_bwd"
    with pytest.raises(gpu_lib.FA2Error):
        gpu_lib.fa2_bwd_noalloc(*(dev["q"],) * 9, B, H, N + 1, d, 0.1, 1, -1, -1)
