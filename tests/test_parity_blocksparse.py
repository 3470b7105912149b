"""Block-sparse attention: HIP forward and backward through the C ABI against
the fp64 oracle (dense masks plus a 128 x 128 block mask).

* small problems with random block masks that leave whole query rows without
  a visible key (O = 0, LSE = -inf, zero gradients), every mask kind, d = 64
  and 128, ragged N: every output element checked;
* an all-ones mask is bitwise the dense entry points;
* a mask shared across the batch (stride 0) equals the same mask repeated;
* the full block-sparse workload (B=4, H=32, N=8192, d=128, causal, band +
  global + 10 % random blocks) in the benchmark's launch configuration: 256
  seeded rows plus edge rows for O, LSE and dQ, key rows of two heads for dK, dV.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import TOL_GRAD_REL, TOL_LSE, TOL_O_BF16, max_abs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu

MASKS = {
    "full": (False, (-1, -1), False),
    "causal": (True, (-1, -1), False),
    "window_150_20": (False, (150, 20), False),
    "causal_window_alibi": (True, (200, 0), True),
    "alibi_noncausal": (False, (-1, -1), True),
}


def random_mask(B, H, N, seed, density=0.5):
    nb = -(-N // 128)
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.random((B, H, nb, nb)) < density).astype(np.uint8))


def run(fa2, dev, mask_d, slopes, scale, causal, window):
    sl = None if slopes is None else slopes.cuda()
    out, lse = fa2.flash_attn_blocksparse_fwd(dev["q"], dev["k"], dev["v"], mask_d, scale, causal, window, sl)
    g = fa2.flash_attn_blocksparse_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, mask_d, scale, causal,
                                       window, sl)
    torch.cuda.synchronize()
    return (out, lse) + tuple(g)


def check_full(fa2, B, H, N, d, causal, window, alibi, seed):
    t = workloads.make_inputs(B, H, N, d, "bf16", seed, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    mask = random_mask(B, H, N, seed + 1)
    slopes = workloads.alibi_slopes(H) if alibi else None
    sl = None if slopes is None else slopes.numpy()
    out, lse, dq, dk, dv = run(fa2, dev, mask.cuda(), slopes, scale_of(d), causal, window)
    o_ref, lse_ref = oracle.blocksparse_forward(t["q"], t["k"], t["v"], mask.numpy(), scale_of(d), causal, window, sl)
    g_ref = oracle.blocksparse_backward(t["q"], t["k"], t["v"], t["dout"], mask.numpy(), scale_of(d), causal, window,
                                        sl)
    lse_np = lse.cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_np), empty), "rows without a visible key must get LSE = -inf"
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse_np[~empty], lse_ref[~empty])
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  empty rows {int(empty.sum())}  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg
    return int(empty.sum())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("N", [300, 129])
def test_small_block_sparse(gpu_lib, N, mask, d):
    causal, window, alibi = MASKS[mask]
    say(f"blocksparse small N={N} mask={mask} d={d}")
    check_full(gpu_lib, 2, 3, N, d, causal, window, alibi, seed=71 + d + N)


def test_rows_without_visible_keys_are_exercised(gpu_lib):
    say("blocksparse empty rows")
    assert check_full(gpu_lib, 2, 3, 384, 128, True, (-1, -1), False, seed=75) > 0


@pytest.mark.parametrize("d", [64, 128])
def test_all_ones_mask_bitwise_matches_dense(gpu_lib, d):
    fa2 = gpu_lib
    B, H, N = 2, 3, 333
    say(f"blocksparse all-ones vs dense d={d}")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=76, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    sl = workloads.alibi_slopes(H).cuda()
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale_of(d), True, (100, 0), sl)
    g = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale_of(d), True, (100, 0), sl)
    ones = torch.ones((1, 1, 3, 3), dtype=torch.uint8, device="cuda")
    out_s, lse_s = fa2.flash_attn_blocksparse_fwd(dev["q"], dev["k"], dev["v"], ones, scale_of(d), True, (100, 0), sl)
    g_s = fa2.flash_attn_blocksparse_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out_s, lse_s, ones, scale_of(d),
                                         True, (100, 0), sl)
    torch.cuda.synchronize()
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)
    for a, b in zip(g, g_s):
        assert torch.equal(a, b)


def test_shared_mask_equals_repeated_mask(gpu_lib):
    fa2 = gpu_lib
    B, H, N, d = 3, 2, 400, 64
    say("blocksparse shared vs repeated mask")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=77, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    shared = random_mask(1, H, N, 78).cuda()
    full = shared.expand(B, H, -1, -1).contiguous()
    a = run(fa2, dev, shared, None, scale_of(d), False, (-1, -1))
    b = run(fa2, dev, full, None, scale_of(d), False, (-1, -1))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_full_size_block_sparse_workload_sampled(gpu_lib):
    w = workloads.SPARSE_WORKLOADS[7]
    say(f"blocksparse full size: {w.describe()}")
    t = workloads.make_inputs(w.B, w.H, w.N, w.d, "bf16", seed=w.number, with_dout=True)
    mask = workloads.sparse_block_mask(w.H, w.N, w.local, w.global_blocks, w.density, seed=w.number)
    dev = {k: v.cuda() for k, v in t.items()}
    out, lse, dq, dk, dv = run(gpu_lib, dev, mask.cuda(), None, w.scale, w.causal, w.window)
    rows = workloads.sample_query_rows(w.B, w.H, w.N, 256, seed=1000 + w.number)
    edges = [(b, h, i) for b, h in ((0, 0), (w.B - 1, w.H - 1)) for i in (0, 127, 128, w.N - 1)]
    rows = np.concatenate([rows, np.array(edges, dtype=np.int64)])
    keys = workloads.sample_key_rows(w.B, w.H, w.N, 32, max_heads=2, seed=2000 + w.number)
    full_mask = mask.expand(w.B, -1, -1, -1).numpy()
    o_ref, lse_ref = oracle.blocksparse_forward_rows(t["q"], t["k"], t["v"], full_mask, rows, w.scale, w.causal)
    dq_ref, dk_ref, dv_ref = oracle.blocksparse_backward_sampled(t["q"], t["k"], t["v"], t["dout"], full_mask, rows,
                                                                 keys, w.scale, w.causal)
    b, h, i = (torch.from_numpy(rows[:, c]).cuda() for c in range(3))
    kb, kh, kj = (torch.from_numpy(keys[:, c]).cuda() for c in range(3))
    eo = max_abs(to_np(out[b, i, h]), o_ref)
    el = max_abs(lse[b, h, i].cpu().numpy(), lse_ref)
    edq = rel_to_max(to_np(dq[b, i, h]), dq_ref)
    edk = rel_to_max(to_np(dk[kb, kj, kh]), dk_ref)
    edv = rel_to_max(to_np(dv[kb, kj, kh]), dv_ref)
    say(f"  O {eo:.3e} LSE {el:.3e} dQ {edq:.3e} dK {edk:.3e} dV {edv:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(edq, edk, edv) <= TOL_GRAD_REL
