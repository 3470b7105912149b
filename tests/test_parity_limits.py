"""The hot path at the edges of its supported shapes, through the C ABI, against the
fp64 oracle on sampled rows:

* H * d at the 2^22 ceiling (d = 128, H = 32768; a 17-token ragged sequence), where a
  128-row tile spans 2^30 bytes of 32-bit row offsets;
* a dense causal sequence of 65536 tokens;
* a block-sparse sequence of 65536 tokens, the longest the per-workgroup tile list
  holds.

Query rows are checked against the definition (O, LSE, dQ). Key rows need every row
of their head in the oracle, so at N = 65536 dK and dV are checked by identities that
hold at any size instead: rows of P sum to one, so sum_j dV_j = sum_i dO_i over the
rows that see a key, and rows of dS sum to zero, so sum_j dK_j = 0 (per head and
column). The bf16 rounding of each dK_j, dV_j bounds how far the sums may stray:
2^-9 of the sum of their magnitudes; the tests allow twice that.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import (TOL_GRAD_REL, TOL_LSE, TOL_O_BF16, gather_lse, gather_rows, max_abs, rel_to_max, say,
                          scale_of, to_np)

pytestmark = pytest.mark.gpu


def column_sum_identities(dk, dv, dout, H):
    """Worst |sum_j dK_j| and |sum_j dV_j - sum_i dO_i| per head and column, each over
    2^-8 * sum_j |dK_j| (or |dV_j|) + 1e-3: twice what rounding every element to bf16 can
    add up to, dO being exact bf16 input (every row of dout sees at least one key here)."""
    worst = 0.0
    for h in range(H):
        k_h = dk[0, :, h, :].double()
        v_h = dv[0, :, h, :].double()
        o_h = dout[0, :, h, :].double()
        rk = k_h.sum(0).abs() / (2.0 ** -8 * k_h.abs().sum(0) + 1e-3)
        rv = (v_h.sum(0) - o_h.sum(0)).abs() / (2.0 ** -8 * v_h.abs().sum(0) + 1e-3)
        worst = max(worst, float(rk.max()), float(rv.max()))
    return worst


def test_heads_times_d_at_the_limit(gpu_lib):
    B, H, N, d = 1, 32768, 17, 128  # H * d = 2^22
    sc = scale_of(d)
    say(f"limits: B={B} H={H} N={N} d={d} causal")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=90, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], sc, True, (-1, -1), None)
    dq, dk, dv = gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, sc, True, (-1, -1),
                                        None, True)
    torch.cuda.synchronize()
    rows = np.concatenate([workloads.sample_query_rows(B, H, N, 256, seed=91),
                           np.array([[0, 0, 0], [0, H - 1, N - 1], [0, H // 2, N - 1]], dtype=np.int64)])
    keys = workloads.sample_key_rows(B, H, N, 2 * N, max_heads=2, seed=92)
    keys = np.concatenate([keys, np.array([[0, H - 1, 0], [0, H - 1, N - 1]], dtype=np.int64)])
    o_ref, lse_ref = oracle.attention_forward_rows(t["q"], t["k"], t["v"], rows, sc, True)
    gq, gk, gv = oracle.attention_backward_sampled(t["q"], t["k"], t["v"], t["dout"], rows, keys, sc, True)
    eo = max_abs(gather_rows(to_np(out), rows), o_ref)
    el = max_abs(gather_lse(lse.cpu().numpy(), rows), lse_ref)
    dq_np, dk_np, dv_np = (to_np(x) for x in (dq, dk, dv))
    eg = [rel_to_max(dq_np[rows[:, 0], rows[:, 2], rows[:, 1]], gq),
          rel_to_max(dk_np[keys[:, 0], keys[:, 2], keys[:, 1]], gk),
          rel_to_max(dv_np[keys[:, 0], keys[:, 2], keys[:, 1]], gv)]
    say(f"  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL


def test_dense_causal_sequence_of_65536_tokens(gpu_lib):
    B, H, N, d = 1, 2, 65536, 128
    sc = scale_of(d)
    say(f"limits: B={B} H={H} N={N} d={d} causal")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=93, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    out, lse = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], sc, True, (-1, -1), None)
    dq, dk, dv = gpu_lib.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, sc, True, (-1, -1),
                                        None, True)
    torch.cuda.synchronize()
    rows = np.concatenate([workloads.sample_query_rows(B, H, N, 128, seed=94),
                           np.array([[0, 0, 0], [0, 1, N - 1], [0, 1, 32768]], dtype=np.int64)])
    o_ref, lse_ref = oracle.attention_forward_rows(t["q"], t["k"], t["v"], rows, sc, True)
    gq, _, _ = oracle.attention_backward_sampled(t["q"], t["k"], t["v"], t["dout"], rows, np.zeros((0, 3), np.int64),
                                                 sc, True)
    eo = max_abs(gather_rows(to_np(out), rows), o_ref)
    el = max_abs(gather_lse(lse.cpu().numpy(), rows), lse_ref)
    eq = rel_to_max(to_np(dq)[rows[:, 0], rows[:, 2], rows[:, 1]], gq)
    ident = column_sum_identities(dk.cpu(), dv.cpu(), t["dout"], H)
    say(f"  O {eo:.3e}  LSE {el:.3e}  dQ {eq:.3e}  column-sum identities {ident:.3f} of the bound")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE and eq <= TOL_GRAD_REL
    assert ident <= 1.0


def test_block_sparse_sequence_of_65536_tokens(gpu_lib):
    B, H, N, d = 1, 1, 65536, 64
    sc = scale_of(d)
    mask = workloads.sparse_block_mask(H, N, local=1, global_blocks=1, density=0.02, seed=95)
    say(f"limits: block-sparse B={B} H={H} N={N} d={d} causal, {int(mask.sum())} active blocks")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=96, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    m_dev = mask.cuda()
    out, lse = gpu_lib.flash_attn_blocksparse_fwd(dev["q"], dev["k"], dev["v"], m_dev, sc, True, (-1, -1), None)
    dq, dk, dv = gpu_lib.flash_attn_blocksparse_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, m_dev, sc,
                                                    True, (-1, -1), None)
    torch.cuda.synchronize()
    full_mask = mask.numpy()
    rows = np.concatenate([workloads.sample_query_rows(B, H, N, 128, seed=97),
                           np.array([[0, 0, 0], [0, 0, N - 1], [0, 0, 128]], dtype=np.int64)])
    o_ref, lse_ref = oracle.blocksparse_forward_rows(t["q"], t["k"], t["v"], full_mask, rows, sc, True)
    gq, _, _ = oracle.blocksparse_backward_sampled(t["q"], t["k"], t["v"], t["dout"], full_mask, rows,
                                                   np.zeros((0, 3), np.int64), sc, True)
    eo = max_abs(gather_rows(to_np(out), rows), o_ref)
    el = max_abs(gather_lse(lse.cpu().numpy(), rows), lse_ref)
    eq = rel_to_max(to_np(dq)[rows[:, 0], rows[:, 2], rows[:, 1]], gq)
    ident = column_sum_identities(dk.cpu(), dv.cpu(), t["dout"], H)  # the diagonal block is always on
    say(f"  O {eo:.3e}  LSE {el:.3e}  dQ {eq:.3e}  column-sum identities {ident:.3f} of the bound")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE and eq <= TOL_GRAD_REL
    assert ident <= 1.0
