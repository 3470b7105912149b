"""A seeded sweep over shapes and options: HIP forward and backward through the C ABI
against the fp64 oracle, every output element checked.

Each case draws B, H, N (1..700, so ragged tails and single-tile problems occur), d,
causal, the window (none, left only, right only, both), ALiBi and a dropout rate from
its own seed, so a failure names a reproducible case. Packed batches (1-6 sequences,
empty ones included) and block-sparse batches (random masks, shared or per batch,
rows left without keys) get their own seeded sweeps. Complements the hand-picked
cases of the other parity files.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import TOL_GRAD_REL, TOL_LSE, TOL_O_BF16, max_abs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu

N_CASES = 64


def draw(case):
    r = np.random.default_rng(5000 + case)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    N = int(r.choice([1, 33, 129, int(r.integers(3, 701)), int(r.integers(3, 701)), int(r.integers(3, 701))]))
    d = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    kind = int(r.integers(0, 4))
    wl = int(r.integers(0, N + 40)) if kind in (1, 3) else -1
    wr = int(r.integers(0, N + 40)) if kind in (2, 3) else -1
    alibi = bool(r.integers(0, 2))
    p = float(r.choice([0.0, 0.0, 0.2]))
    return B, H, N, d, causal, (wl, wr), alibi, p


def given_output(t, out, o_ref, g_ref, sc, causal, window, slopes):
    """The oracle gradients (dq, dk, dv) re-based on D = rowsum(dO * out) for the given out."""
    q, k, do = (t[n].double().numpy() for n in ("q", "k", "dout"))
    B, N, H, _ = q.shape
    dd = np.sum(do * (out - o_ref), axis=-1)  # [B, N, H]
    dq, dk, dv = (g.copy() for g in g_ref)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            s = oracle.logits(q[b, :, h, :], k[b, :, h, :], rows, sc, causal, window[0], window[1],
                              None if slopes is None else float(slopes[h]))
            pm, _ = oracle.softmax_rows(s)
            dq[b, :, h, :] -= sc * dd[b, :, h, None] * (pm @ k[b, :, h, :])
            dk[b, :, h, :] -= sc * (pm.T @ (dd[b, :, h, None] * q[b, :, h, :]))
    return dq, dk, dv


@pytest.mark.parametrize("case", range(N_CASES))
def test_seeded_sweep(gpu_lib, case):
    fa2 = gpu_lib
    B, H, N, d, causal, window, alibi, p = draw(case)
    say(f"sweep case {case}: B={B} H={H} N={N} d={d} causal={causal} window={window} alibi={alibi} p={p}")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=6000 + case, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    slopes = workloads.alibi_slopes(H) if alibi else None
    sl_d = None if slopes is None else slopes.cuda()
    sl = None if slopes is None else slopes.numpy()
    sc = scale_of(d)
    seed, offset = 7000 + case, 3
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], sc, causal, window, sl_d, dropout_p=p, seed=seed,
                                  offset=offset)
    dq, dk, dv = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, sc, causal, window, sl_d,
                                    deterministic=True, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    if p > 0:
        o_ref, lse_ref = oracle.dropout_forward(t["q"], t["k"], t["v"], p, seed, offset, sc, causal, window, sl)
        g_ref = oracle.dropout_backward(t["q"], t["k"], t["v"], t["dout"], p, seed, offset, sc, causal, window, sl)
    else:
        o_ref, lse_ref = oracle.attention_forward(t["q"], t["k"], t["v"], sc, causal, window, sl)
        g_ref = oracle.attention_backward(t["q"], t["k"], t["v"], t["dout"], sc, causal, window, sl)
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    # fa2_bwd takes the forward's output as an input and forms D = rowsum(dO * out) from
    # it, so its reference is the oracle's gradient with that D: dS moves by -P * dD,
    # dQ by -scale * dD * (P K) and dK by -scale * P^T (dD * Q). It matters only where the
    # exact dQ, dK vanish (every row sees a single key) and the rounding of the stored O
    # (scaled by 1/(1-p) under dropout) is all that is left.
    g_ref = given_output(t, to_np(out), o_ref, g_ref, sc, causal, window, sl)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg


# ---------------------------------------------------------------- packed and block-sparse batches

def draw_packed(case):
    r = np.random.default_rng(8000 + case)
    nseq = int(r.integers(1, 7))
    lengths = [int(x) for x in r.choice([1, 2, 31, 33, 128, 129, int(r.integers(1, 400))], size=nseq)]
    if r.integers(0, 4) == 0:
        lengths[int(r.integers(0, nseq))] = 0  # an empty sequence
    H, d = int(r.integers(1, 4)), int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    kind = int(r.integers(0, 4))
    wl = int(r.integers(0, 300)) if kind in (1, 3) else -1
    wr = int(r.integers(0, 300)) if kind in (2, 3) else -1
    return lengths, H, d, causal, (wl, wr), bool(r.integers(0, 2))


@pytest.mark.parametrize("case", range(24))
def test_seeded_packed_sweep(gpu_lib, case):
    fa2 = gpu_lib
    lengths, H, d, causal, window, alibi = draw_packed(case)
    T = sum(lengths)
    say(f"packed sweep case {case}: lengths={lengths} H={H} d={d} causal={causal} window={window} alibi={alibi}")
    if T == 0:
        lengths[0] = 5
        T = 5
    t = workloads.make_varlen_inputs(T, H, d, "bf16", seed=9000 + case, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    cu = workloads.cu_seqlens_from_lengths(lengths)
    slopes = workloads.alibi_slopes(H) if alibi else None
    sl = None if slopes is None else slopes.numpy()
    sc = scale_of(d)
    out, lse = fa2.flash_attn_varlen_fwd(dev["q"], dev["k"], dev["v"], cu.cuda(), sc, causal, window,
                                         None if slopes is None else slopes.cuda())
    dq, dk, dv = fa2.flash_attn_varlen_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, cu.cuda(), sc, causal,
                                           window, None if slopes is None else slopes.cuda())
    torch.cuda.synchronize()
    cu_np = cu.numpy()
    o_ref, lse_ref = oracle.varlen_forward(t["q"], t["k"], t["v"], cu_np, sc, causal, window, sl)
    g_ref = oracle.varlen_backward(t["q"], t["k"], t["v"], t["dout"], cu_np, sc, causal, window, sl)
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg


def draw_sparse(case):
    r = np.random.default_rng(9500 + case)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    N = int(r.choice([1, 128, 129, 255, int(r.integers(2, 520))]))
    d = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    kind = int(r.integers(0, 3))
    window = [(-1, -1), (int(r.integers(0, 300)), 0 if causal else int(r.integers(0, 300))),
              (int(r.integers(0, 300)), -1)][kind]
    density = float(r.choice([0.3, 0.6, 1.0]))
    shared = bool(r.integers(0, 2))
    return B, H, N, d, causal, window, bool(r.integers(0, 2)), density, shared


@pytest.mark.parametrize("case", range(24))
def test_seeded_blocksparse_sweep(gpu_lib, case):
    fa2 = gpu_lib
    B, H, N, d, causal, window, alibi, density, shared = draw_sparse(case)
    say(f"block-sparse sweep case {case}: B={B} H={H} N={N} d={d} causal={causal} window={window} alibi={alibi} "
        f"density={density} shared={shared}")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=9700 + case, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    nb = -(-N // 128)
    rng = np.random.default_rng(9900 + case)
    mask = torch.from_numpy((rng.random((1 if shared else B, H, nb, nb)) < density).astype(np.uint8))
    slopes = workloads.alibi_slopes(H) if alibi else None
    sl = None if slopes is None else slopes.numpy()
    sc = scale_of(d)
    sl_d = None if slopes is None else slopes.cuda()
    out, lse = fa2.flash_attn_blocksparse_fwd(dev["q"], dev["k"], dev["v"], mask.cuda(), sc, causal, window, sl_d)
    dq, dk, dv = fa2.flash_attn_blocksparse_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, mask.cuda(), sc,
                                                causal, window, sl_d)
    torch.cuda.synchronize()
    full_mask = mask.expand(B, -1, -1, -1).numpy()
    o_ref, lse_ref = oracle.blocksparse_forward(t["q"], t["k"], t["v"], full_mask, sc, causal, window, sl)
    g_ref = oracle.blocksparse_backward(t["q"], t["k"], t["v"], t["dout"], full_mask, sc, causal, window, sl)
    lse_np = lse.cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_np), empty)
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse_np[~empty], lse_ref[~empty])
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  empty rows {int(empty.sum())}  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg
