"""Dropout on the attention weights: HIP forward and backward through the C ABI
against the fp64 oracle (keep matrix from Philox4x64-10, weights scaled by 1/(1-p)).

* the keep matrix itself, bit for bit, in each of the three kernels, read off
  structured inputs: Q = 0 and V = identity make O_ij non-zero iff weight
  (i, j) is kept (forward); dO = identity does the same for dV^T (key-block
  pass); K = identity with V = dO = e_0 makes the sign of dQ_ij say whether
  (i, j) was kept (dQ pass);
* small problems, every mask kind, d = 64 and 128, ragged N, two rates: every
  output element against the oracle;
* repeatability, independence of the offset, and p = 0 equal to the dense path;
* the B=4, H=32, N=8192, d=128 causal shape at p = 0.1 in the benchmark's launch
  configuration: 256 seeded rows plus edge rows for O, LSE and dQ, key rows of
  two heads for dK and dV.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import dropout as od
from parity_utils import TOL_GRAD_REL, TOL_LSE, TOL_O_BF16, max_abs, rel_to_max, say, scale_of, to_np

pytestmark = pytest.mark.gpu

MASKS = {
    "full": (False, (-1, -1), False),
    "causal": (True, (-1, -1), False),
    "window_70_20": (False, (70, 20), False),
    "causal_window_alibi": (True, (200, 0), True),
}


def keep_matrix(bh, N, p, seed, offset):
    return od.keep_rows(bh, np.arange(N), N, p, seed, offset)


def run(fa2, dev, slopes, scale, causal, window, p, seed, offset):
    sl = None if slopes is None else slopes.cuda()
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale, causal, window, sl, dropout_p=p, seed=seed,
                                  offset=offset)
    g = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale, causal, window, sl,
                           dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return (out, lse) + tuple(g)


def structured(B, H, N, d, q=None, k=None, v=None, dout=None, seed=0):
    """bf16 device tensors [B, N, H, d]: N(0,1) unless a [N, d] pattern is given (then shared by all heads)."""
    t = workloads.make_inputs(B, H, N, d, "bf16", seed, with_dout=True)
    for name, pat in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if pat is not None:
            t[name] = torch.from_numpy(np.broadcast_to(pat[None, :, None, :], (B, N, H, d)).copy()).to(torch.bfloat16)
    return t, {k_: v_.cuda() for k_, v_ in t.items()}


# ---------------------------------------------------------------- the keep matrix, bit for bit

# (seed, offset): small values, and a full 64-bit seed with the largest offset
SEEDS = [(1234, 5), (0xFEDCBA9876543210, 2**32 - 1)]


@pytest.mark.parametrize("so", SEEDS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_keep_matrix_is_bitwise_the_oracles(gpu_lib, d, causal, so):
    B, H, N, p = 2, 3, d, 0.5
    seed, offset = so
    say(f"dropout keep matrix, forward d={d} causal={causal}")
    _, dev = structured(B, H, N, d, q=np.zeros((N, d)), v=np.eye(N, d))
    out, _ = gpu_lib.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale_of(d), causal, dropout_p=p, seed=seed,
                                    offset=offset)
    o = to_np(out)
    vis = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            z = keep_matrix(b * H + h, N, p, seed, offset)
            got = o[b, :, h, :] != 0
            assert np.array_equal(got[vis], z[vis]), f"(b, h) = ({b}, {h})"
            assert not got[~vis].any()


@pytest.mark.parametrize("so", SEEDS)
@pytest.mark.parametrize("d", [64, 128])
def test_key_block_pass_keep_matrix_is_bitwise_the_oracles(gpu_lib, d, so):
    B, H, N, p = 2, 3, d, 0.5
    seed, offset = so
    say(f"dropout keep matrix, dK/dV pass d={d}")
    _, dev = structured(B, H, N, d, q=np.zeros((N, d)), dout=np.eye(N, d), seed=3)
    _, _, _, _, dv = run(gpu_lib, dev, None, scale_of(d), False, (-1, -1), p, seed, offset)
    g = to_np(dv)
    for b in range(B):
        for h in range(H):
            z = keep_matrix(b * H + h, N, p, seed, offset)
            # dV_j[i] = P_ij Z_ij dO_i[i] / (1 - p) with P_ij = 1/N: non-zero iff (i, j) kept
            assert np.array_equal(g[b, :, h, :].T != 0, z), f"(b, h) = ({b}, {h})"


@pytest.mark.parametrize("so", SEEDS)
@pytest.mark.parametrize("d", [64, 128])
def test_dq_pass_keep_matrix_is_bitwise_the_oracles(gpu_lib, d, so):
    B, H, N, p = 2, 3, d, 0.5
    seed, offset = so
    say(f"dropout keep matrix, dQ pass d={d}")
    e0 = np.zeros((N, d))
    e0[:, 0] = 1.0
    _, dev = structured(B, H, N, d, q=np.zeros((N, d)), k=np.eye(N, d), v=e0, dout=e0)
    _, _, dq, _, _ = run(gpu_lib, dev, None, scale_of(d), False, (-1, -1), p, seed, offset)
    g = to_np(dq)
    for b in range(B):
        for h in range(H):
            z = keep_matrix(b * H + h, N, p, seed, offset)
            # dS_ij = (Z_ij / (1 - p) - D_i) / N with 0 < D_i < 1 / (1 - p): positive iff kept
            assert np.all(g[b, :, h, :] != 0)
            assert np.array_equal(g[b, :, h, :] > 0, z), f"(b, h) = ({b}, {h})"


# Far from the origin: a causal window of 128 keys (window_left = 127) with uniform weights
# (q = 0) and one-hot rows by position mod 128 make every output element carry exactly one
# keep bit, so whole keep matrices at N = 2048 (generator groups up to 127, rows up to 2047)
# are compared bit for bit in all three kernels.
NFAR, DFAR, WFAR = 2048, 128, 127
FAR_SEED, FAR_OFFSET = 0x0123456789ABCDEF, 2**31 + 12345


def residue_rows(N, d):
    r = np.zeros((N, d))
    r[np.arange(N), np.arange(N) % d] = 1.0
    return r


def far_run(gpu_lib, **pats):
    _, dev = structured(1, 2, NFAR, DFAR, seed=5, **pats)
    return run(gpu_lib, dev, None, scale_of(DFAR), True, (WFAR, 0), 0.5, FAR_SEED, FAR_OFFSET)


def key_of_residue(i, c):
    """The key of row i's window [i - 127, i] congruent to c mod 128, or -1."""
    j = i - ((i - c) % 128)
    return j if j >= 0 else -1


def test_forward_keep_matrix_far_from_the_origin(gpu_lib):
    say("dropout keep matrix, forward, N=2048 window 128")
    out, _, _, _, _ = far_run(gpu_lib, q=np.zeros((NFAR, DFAR)), v=residue_rows(NFAR, DFAR))
    o = to_np(out)
    for h in range(2):
        z = keep_matrix(h, NFAR, 0.5, FAR_SEED, FAR_OFFSET)
        i, c = np.meshgrid(np.arange(NFAR), np.arange(DFAR), indexing="ij")
        j = i - ((i - c) % 128)
        want = np.where(j >= 0, z[i, np.maximum(j, 0)], False)
        assert np.array_equal(o[0, :, h, :] != 0, want), f"head {h}"


def test_key_block_pass_keep_matrix_far_from_the_origin(gpu_lib):
    say("dropout keep matrix, dK/dV pass, N=2048 window 128")
    _, _, _, _, dv = far_run(gpu_lib, q=np.zeros((NFAR, DFAR)), dout=residue_rows(NFAR, DFAR))
    g = to_np(dv)
    for h in range(2):
        z = keep_matrix(h, NFAR, 0.5, FAR_SEED, FAR_OFFSET)
        j, c = np.meshgrid(np.arange(NFAR), np.arange(DFAR), indexing="ij")
        i = j + ((c - j) % 128)  # the query of key j's window [j, j + 127] congruent to c
        want = np.where(i < NFAR, z[np.minimum(i, NFAR - 1), j], False)
        # dV_j[c] = P Z / (1 - p) for that query: non-zero iff (query, key) kept
        assert np.array_equal(g[0, :, h, :] != 0, want), f"head {h}"


def test_dq_pass_keep_matrix_far_from_the_origin(gpu_lib):
    say("dropout keep matrix, dQ pass, N=2048 window 128")
    e0 = np.zeros((NFAR, DFAR))
    e0[:, 0] = 1.0
    _, _, dq, _, _ = far_run(gpu_lib, q=np.zeros((NFAR, DFAR)), k=residue_rows(NFAR, DFAR), v=e0, dout=e0)
    g = to_np(dq)
    for h in range(2):
        z = keep_matrix(h, NFAR, 0.5, FAR_SEED, FAR_OFFSET)
        checked = 0
        for i in range(NFAR):
            lo = max(0, i - WFAR)
            kept = int(z[i, lo:i + 1].sum())
            if kept == 0 or kept == i + 1 - lo:
                continue  # D equals every kept weight's value (or none is kept): dS is 0
            for c in range(DFAR):
                j = key_of_residue(i, c)
                # dQ_i[c] = scale dS_ij = scale P (Z / (1 - p) - D_i), 0 < D_i < 1 / (1 - p)
                assert (g[0, i, h, c] > 0) == (j >= 0 and bool(z[i, j])), f"head {h} row {i} col {c}"
                assert j >= 0 or g[0, i, h, c] == 0
            checked += 1
        assert checked > NFAR - 20


# ---------------------------------------------------------------- values against the oracle

def check_small(fa2, B, H, N, d, causal, window, alibi, p, seed, o_tol=TOL_O_BF16):
    t = workloads.make_inputs(B, H, N, d, "bf16", seed, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    slopes = workloads.alibi_slopes(H) if alibi else None
    sl = None if slopes is None else slopes.numpy()
    ds, doff = 1000 + seed, 17
    out, lse, dq, dk, dv = run(fa2, dev, slopes, scale_of(d), causal, window, p, ds, doff)
    o_ref, lse_ref = oracle.dropout_forward(t["q"], t["k"], t["v"], p, ds, doff, scale_of(d), causal, window, sl)
    g_ref = oracle.dropout_backward(t["q"], t["k"], t["v"], t["dout"], p, ds, doff, scale_of(d), causal, window, sl)
    eo = max_abs(to_np(out), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    eg = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O {eo:.3e}  LSE {el:.3e}  grads {eg[0]:.3e} {eg[1]:.3e} {eg[2]:.3e}")
    assert eo <= o_tol and el <= TOL_LSE
    assert max(eg) <= TOL_GRAD_REL, eg


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("N", [300, 129])
def test_small_dropout(gpu_lib, N, mask, d, p):
    causal, window, alibi = MASKS[mask]
    say(f"dropout small N={N} mask={mask} d={d} p={p}")
    check_small(gpu_lib, 2, 3, N, d, causal, window, alibi, p, seed=81 + d + N)


@pytest.mark.parametrize("p", [1e-6, 0.99, 0.999])
@pytest.mark.parametrize("N", [1, 17, 200])
def test_extreme_rates_and_short_sequences(gpu_lib, N, p):
    # p = 1e-6 keeps every weight (threshold 256) but still rescales; p = 0.99 keeps
    # 3 in 256 (threshold 3), so most short rows are all-dropped (O = 0, LSE
    # unchanged); p = 0.999 has threshold 0 and drops every weight.
    # The kept weights are scaled by 1/(1-p), so O and its bf16 rounding error grow
    # by that factor: the absolute O bound is scaled with it.
    say(f"dropout edge N={N} p={p}")
    check_small(gpu_lib, 2, 2, N, 128, True, (-1, -1), False, p, seed=91 + N, o_tol=TOL_O_BF16 / (1 - p))


def test_repeatable_offset_sensitive_and_p_zero_is_dense(gpu_lib):
    fa2 = gpu_lib
    B, H, N, d = 2, 2, 257, 128
    say("dropout repeatability / offset / p = 0")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=88, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    a = run(fa2, dev, None, scale_of(d), True, (-1, -1), 0.2, 5, 0)
    b = run(fa2, dev, None, scale_of(d), True, (-1, -1), 0.2, 5, 0)
    c = run(fa2, dev, None, scale_of(d), True, (-1, -1), 0.2, 5, 1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])  # new keep matrix, same LSE
    # p = 0 through the dropout entry points is the dense computation
    z_out, z_lse = torch.empty_like(dev["q"]), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    zg = [torch.empty_like(dev["q"]) for _ in range(3)]
    ws = torch.empty(fa2.fa2_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    fa2.fa2_fwd_dropout(dev["q"], dev["k"], dev["v"], z_out, z_lse, B, H, N, d, scale_of(d), 1, -1, -1, None, 0.0, 5, 0)
    fa2.fa2_bwd_dropout(dev["q"], dev["k"], dev["v"], z_out, z_lse, dev["dout"], *zg, ws, ws.numel(), B, H, N, d,
                        scale_of(d), 1, -1, -1, None, 0.0, 5, 0)
    z = (z_out, z_lse) + tuple(zg)
    out, lse = fa2.flash_attn_fwd(dev["q"], dev["k"], dev["v"], scale_of(d), True)
    g = fa2.flash_attn_bwd(dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, scale_of(d), True)
    torch.cuda.synchronize()
    for x, y in zip(z, (out, lse) + tuple(g)):
        assert torch.equal(x, y)


def test_full_size_dropout_sampled(gpu_lib):
    B, H, N, d, p, seed, offset = 4, 32, 8192, 128, 0.1, 2024, 0
    say(f"dropout full size: B={B} H={H} N={N} d={d} causal p={p}")
    t = workloads.make_inputs(B, H, N, d, "bf16", seed=3, with_dout=True)
    dev = {k: v.cuda() for k, v in t.items()}
    out, lse, dq, dk, dv = run(gpu_lib, dev, None, scale_of(d), True, (-1, -1), p, seed, offset)
    rows = workloads.sample_query_rows(B, H, N, 256, seed=1003)
    edges = [(b, h, i) for b, h in ((0, 0), (B - 1, H - 1)) for i in (0, 15, 16, 4095, N - 1)]
    rows = np.concatenate([rows, np.array(edges, dtype=np.int64)])
    keys = workloads.sample_key_rows(B, H, N, 32, max_heads=2, seed=2003)
    args = (p, seed, offset, scale_of(d), True)
    o_ref, lse_ref = oracle.dropout_forward_rows(t["q"], t["k"], t["v"], rows, *args)
    dq_ref, dk_ref, dv_ref = oracle.dropout_backward_sampled(t["q"], t["k"], t["v"], t["dout"], rows, keys, *args)
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
