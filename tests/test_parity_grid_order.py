"""Parity at head counts that take the XCD-aware grid orders, every output element
against the fp64 oracle.

The kernels map a workgroup id to (head, block) in one of three ways, chosen by the
number of (batch, head) pairs bh: head-fastest in general; when bh is a multiple of
32, groups of 4 heads x, x+8, x+16, x+24 per XCD (the backward passes); when bh is a
multiple of 16, pairs of neighbouring heads per XCD (the forward). The small problems
of the other parity files have bh below 8 and so take only the first. A mistake in
the other two would leave some block unwritten or write it twice; these cases cover
each of them for the dense, packed and block-sparse entry points, with a ragged last
block and several query and key blocks per head.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import TOL_GRAD_REL, TOL_LSE, TOL_O_BF16, gpu_inputs, max_abs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu

# (B, H): bh = 16 (forward pairs only), 32 (both orders), 48 (three forward pair
# groups), 64 (two backward groups per XCD).
HEADS = [(2, 8), (1, 32), (3, 16), (4, 16)]
MASKS = {
    "full": (False, (-1, -1), False),
    "causal": (True, (-1, -1), False),
    "causal_window_alibi": (True, (100, 0), True),
}


@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("heads", HEADS, ids=lambda bh: f"B{bh[0]}H{bh[1]}")
def test_dense_forward_and_backward(gpu_lib, heads, mask):
    B, H = heads
    N, d = 333, 128
    causal, window, alibi = MASKS[mask]
    say(f"grid order dense B={B} H={H} N={N} d={d} mask={mask}")
    cpu, dev, slopes = gpu_inputs(B, H, N, d, "bf16", seed=400 + B * H, with_dout=True, alibi=alibi)
    sl_d = None if slopes is None else slopes.cuda()
    sl = None if slopes is None else slopes.numpy()
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale_of(d), causal, window, sl_d)
    dq, dk, dv = gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale_of(d), causal,
                                        window, sl_d, False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], scale_of(d), causal, window, sl)
    g_ref = oracle.attention_backward(cpu["q"], cpu["k"], cpu["v"], cpu["dout"], scale_of(d), causal, window, sl)
    eo, el = max_abs(to_np(out), o_ref), max_abs(to_np(lse), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg


def test_dense_forward_d64(gpu_lib):
    B, H, N, d = 2, 16, 333, 64
    say(f"grid order dense B={B} H={H} N={N} d={d} causal")
    cpu, dev, _ = gpu_inputs(B, H, N, d, "bf16", seed=431)
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale_of(d), True, (-1, -1), None)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(cpu["q"], cpu["k"], cpu["v"], scale_of(d), True)
    assert max_abs(to_np(out), o_ref) <= TOL_O_BF16 and max_abs(to_np(lse), lse_ref) <= TOL_LSE


@pytest.mark.parametrize("H", [16, 32])
def test_packed_batch(gpu_lib, H):
    """Packed batches map heads alone (bh = H), so H = 16 and 32 take the pair order."""
    lengths, d = [300, 0, 129, 64, 255], 128
    say(f"grid order packed H={H} lengths={lengths}")
    T = int(sum(lengths))
    cpu = workloads.make_varlen_inputs(T, H, d, "bf16", 440 + H, with_dout=True)
    cu = workloads.cu_seqlens_from_lengths(lengths)
    dev = {k: v.cuda() for k, v in cpu.items()}
    cu_d = cu.cuda()
    out, lse = gpu_lib.flash_attn_varlen_fwd(dev["q"], dev["k"], dev["v"], cu_d, scale_of(d), True, (-1, -1), None)
    g = gpu_lib.flash_attn_varlen_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, cu_d, scale_of(d), True,
                                      (-1, -1), None)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.varlen_forward(cpu["q"], cpu["k"], cpu["v"], cu.numpy(), scale_of(d), True, (-1, -1), None)
    g_ref = oracle.varlen_backward(cpu["q"], cpu["k"], cpu["v"], cpu["dout"], cu.numpy(), scale_of(d), True,
                                   (-1, -1), None)
    eo, el = max_abs(to_np(out), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip(g, g_ref)]
    say(f"  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg


@pytest.mark.parametrize("heads", [(2, 8), (1, 32)], ids=lambda bh: f"B{bh[0]}H{bh[1]}")
def test_block_sparse(gpu_lib, heads):
    B, H = heads
    N, d = 300, 128
    say(f"grid order block-sparse B={B} H={H} N={N}")
    t = workloads.make_inputs(B, H, N, d, "bf16", 450 + B * H, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    nb = -(-N // 128)
    mask = torch.from_numpy((np.random.default_rng(451).random((B, H, nb, nb)) < 0.6).astype(np.uint8))
    out, lse = gpu_lib.flash_attn_blocksparse_fwd(dev["q"], dev["k"], dev["v"], mask.cuda(), scale_of(d), True,
                                                  (-1, -1), None)
    g = gpu_lib.flash_attn_blocksparse_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, mask.cuda(),
                                           scale_of(d), True, (-1, -1), None)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.blocksparse_forward(t["q"], t["k"], t["v"], mask.numpy(), scale_of(d), True, (-1, -1),
                                                None)
    g_ref = oracle.blocksparse_backward(t["q"], t["k"], t["v"], t["dout"], mask.numpy(), scale_of(d), True, (-1, -1),
                                        None)
    lse_np = lse.cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_np), empty)
    eo, el = max_abs(to_np(out), o_ref), max_abs(lse_np[~empty], lse_ref[~empty])
    eg = [rel_to_max(to_np(x), r) for x, r in zip(g, g_ref)]
    say(f"  empty rows {int(empty.sum())}  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg
