"""Variable-length (packed) batches: HIP forward and backward through the C ABI
against the fp64 oracle, which runs every packed sequence as its own problem.

* small ragged batches (empty, length-1, tile-edge and multi-tile sequences),
  every mask kind, d = 64 and 128: every output element checked;
* more than 64 sequences, so the device-side block lookup scans several
  chunks of boundaries;
* equal lengths: bitwise the same as the fixed-length entry points on the same
  tokens (the kernels share every arithmetic step);
* the full packed workload (T = 32768, 12 ragged sequences, H = 32, d = 128,
  causal), in the launch configuration the benchmark times: 256 seeded
  (head, token) rows plus fixed edge rows for O, LSE and dQ, and key rows of
  two heads in three sequences for dK and dV.
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
    "window_37_5": (False, (37, 5), False),
    "causal_window_alibi": (True, (100, 0), True),
    "alibi_noncausal": (False, (-1, -1), True),
}

LENGTHS = {
    "ragged": [300, 0, 1, 17, 128, 129, 64, 255],
    "one": [301],
    "empty_ends": [0, 0, 77, 0],
}


def packed_inputs(lengths, H, d, seed, alibi):
    T = int(sum(lengths))
    cpu = workloads.make_varlen_inputs(T, H, d, "bf16", seed, with_dout=True)
    cu = workloads.cu_seqlens_from_lengths(lengths)
    dev = {k: v.cuda() for k, v in cpu.items()}
    slopes = workloads.alibi_slopes(H) if alibi else None
    return cpu, dev, cu, slopes


def run(fa2, dev, cu, slopes, scale, causal, window):
    sl = None if slopes is None else slopes.cuda()
    cu_d = cu.cuda()
    out, lse = fa2.flash_attn_varlen_fwd(dev["q"], dev["k"], dev["v"], cu_d, scale, causal, window, sl)
    dq, dk, dv = fa2.flash_attn_varlen_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, cu_d, scale, causal,
                                           window, sl)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def check_full(fa2, lengths, H, d, causal, window, alibi, seed):
    cpu, dev, cu, slopes = packed_inputs(lengths, H, d, seed, alibi)
    scale = scale_of(d)
    out, lse, dq, dk, dv = run(fa2, dev, cu, slopes, scale, causal, window)
    sl = None if slopes is None else slopes.numpy()
    o_ref, lse_ref = oracle.varlen_forward(cpu["q"], cpu["k"], cpu["v"], cu.numpy(), scale, causal, window, sl)
    g_ref = oracle.varlen_backward(cpu["q"], cpu["k"], cpu["v"], cpu["dout"], cu.numpy(), scale, causal, window, sl)
    eo, el = max_abs(to_np(out), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O err {eo:.3e}  LSE err {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("lengths", sorted(LENGTHS))
def test_small_packed_batches(gpu_lib, lengths, mask, d):
    causal, window, alibi = MASKS[mask]
    say(f"varlen small lengths={lengths} mask={mask} d={d}")
    check_full(gpu_lib, LENGTHS[lengths], 3, d, causal, window, alibi, seed=61 + d)


def test_more_than_64_sequences(gpu_lib):
    rng = np.random.default_rng(62)
    lengths = rng.integers(0, 40, size=150).tolist()
    say(f"varlen 150 sequences, T={sum(lengths)}")
    check_full(gpu_lib, lengths, 2, 64, True, (-1, -1), False, seed=62)
    check_full(gpu_lib, lengths, 2, 128, False, (9, 3), True, seed=63)


@pytest.mark.parametrize("d", [64, 128])
def test_equal_lengths_bitwise_match_fixed_length(gpu_lib, d):
    fa2 = gpu_lib
    B, H, N = 3, 4, 333
    say(f"varlen equal lengths vs fixed, d={d}")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=64, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    sl = workloads.alibi_slopes(H).cuda()
    scale = scale_of(d)
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, True, (50, 0), sl)
    dq, dk, dv = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale, True, (50, 0), sl)
    cu = workloads.cu_seqlens_from_lengths([N] * B).cuda()
    flat = {k: v.reshape(B * N, H, d) for k, v in dev.items()}
    out_v, lse_v = fa2.flash_attn_varlen_fwd(flat["q"], flat["k"], flat["v"], cu, scale, True, (50, 0), sl)
    g_v = fa2.flash_attn_varlen_bwd(flat["dout"], flat["q"], flat["k"], flat["v"], out_v, lse_v, cu, scale, True,
                                    (50, 0), sl)
    torch.cuda.synchronize()
    assert torch.equal(out_v, out.reshape(B * N, H, d))
    assert torch.equal(lse_v, lse.permute(1, 0, 2).reshape(H, B * N))
    for a, b in zip(g_v, (dq, dk, dv)):
        assert torch.equal(a, b.reshape(B * N, H, d))


def key_rows_for(cu, H, seed):
    """Key rows (h, t) from two seeded heads in three sequences: the longest, the
    shortest and the last one, 12 tokens each (first and last token included)."""
    rng = np.random.default_rng(seed)
    lens = np.diff(cu)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), len(lens) - 1})
    heads = sorted(rng.choice(H, size=2, replace=False).tolist())
    rows = []
    for b in seqs:
        a, e = int(cu[b]), int(cu[b + 1])
        ts = {a, e - 1, *rng.integers(a, e, size=10).tolist()}
        rows += [(h, t) for h in heads for t in sorted(ts)]
    return np.array(rows, dtype=np.int64)


def test_full_size_packed_workload_sampled(gpu_lib):
    w = workloads.VARLEN_WORKLOADS[6]
    say(f"varlen full size: {w.describe()}")
    t = workloads.varlen_workload_inputs(w)
    cu = t["cu_seqlens"].numpy()
    dev = {k: t[k].cuda() for k in ("q", "k", "v", "dout")}
    out, lse, dq, dk, dv = run(gpu_lib, dev, t["cu_seqlens"], None, w.scale, w.causal, w.window)
    rows = workloads.sample_varlen_rows(w.total, w.H, 256, seed=1000 + w.number)
    edges = [(h, int(x)) for h in (0, w.H - 1) for x in (cu[0], cu[1] - 1, cu[1], cu[-2], cu[-1] - 1)]
    rows = np.concatenate([rows, np.array(edges, dtype=np.int64)])
    keys = key_rows_for(cu, w.H, seed=2000 + w.number)
    o_ref, lse_ref = oracle.varlen_forward_rows(t["q"], t["k"], t["v"], cu, rows, w.scale, w.causal, w.window)
    dq_ref, dk_ref, dv_ref = oracle.varlen_backward_sampled(t["q"], t["k"], t["v"], t["dout"], cu, rows, keys,
                                                            w.scale, w.causal, w.window)
    h, tok = (torch.from_numpy(rows[:, c]).cuda() for c in (0, 1))
    kh, kt = (torch.from_numpy(keys[:, c]).cuda() for c in (0, 1))
    eo = max_abs(to_np(out[tok, h]), o_ref)
    el = max_abs(lse[h, tok].cpu().numpy(), lse_ref)
    edq = rel_to_max(to_np(dq[tok, h]), dq_ref)
    edk = rel_to_max(to_np(dk[kt, kh]), dk_ref)
    edv = rel_to_max(to_np(dv[kt, kh]), dv_ref)
    say(f"  O {eo:.3e} LSE {el:.3e} dQ {edq:.3e} dK {edk:.3e} dV {edv:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(edq, edk, edv) <= TOL_GRAD_REL
