"""Pins for the fp64 oracle: it is checked against things other than itself.

* a worked example derived by hand from the definition (tests/golden);
* closed forms (Q = 0 gives the mean of the visible V rows and LSE = ln(count);
  with ALiBi the geometric series);
* the invariants of attention: rows of P sum to 1, constant V, a single key,
  causal row 0, shift invariance in K, permutation equivariance;
* the online-softmax recurrence of "AI基础 | Flash Attention" (section 在线softmax),
  in both the per-block-normalised and the deferred form;
* library routines that share no code with it (torch CPU fp64 scaled dot-product
  attention and autograd) and central finite differences for the gradients;
* planted mistakes: each plausible error in the oracle trips one of the pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_n3.json")


def rnd(B, N, H, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, N, H, d)) for _ in range(4)]


MASKS = [
    dict(causal=False, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(-1, -1), alibi=False),
    dict(causal=False, window_size=(3, 2), alibi=False),
    dict(causal=True, window_size=(4, 0), alibi=True),
    dict(causal=False, window_size=(-1, -1), alibi=True),
    dict(causal=False, window_size=(0, -1), alibi=False),
]


def slopes_for(H, on):
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]) if on else None


# ---------------------------------------------------------------- worked example

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _as_bnhd(rows):
    return np.array(rows, dtype=np.float64)[None, :, None, :]


def check_golden_forward():
    g = _golden()
    q, k, v = _as_bnhd(g["q"]), _as_bnhd(g["k"]), _as_bnhd(g["v"])
    worst = 0.0
    for c in g["cases"]:
        qq = q * c.get("q_multiplier", 1.0)
        al = None if c["alibi"] is None else np.array(c["alibi"])
        o, lse = oracle.attention_forward(qq, k, v, c["scale"], c["causal"], tuple(c["window"]), al)
        worst = max(worst, np.max(np.abs(o[0, :, 0, :] - np.array(c["out"]))),
                    np.max(np.abs(lse[0, 0] - np.array(c["lse"]))))
    return worst


def check_golden_backward():
    g = _golden()
    q, k, v = _as_bnhd(g["q"]), _as_bnhd(g["k"]), _as_bnhd(g["v"])
    bw = g["backward"]
    dq, dk, dv = oracle.attention_backward(q, k, v, _as_bnhd(bw["dout"]), 1.0, False, (-1, -1), None)
    return max(np.max(np.abs(dq[0, :, 0] - np.array(bw["dq"]))),
               np.max(np.abs(dk[0, :, 0] - np.array(bw["dk"]))),
               np.max(np.abs(dv[0, :, 0] - np.array(bw["dv"]))))


def test_golden_worked_example_forward():
    assert check_golden_forward() < 1e-14


def test_golden_worked_example_backward():
    assert check_golden_backward() < 1e-14


# ---------------------------------------------------------------- closed forms (Q = 0)

def check_q0_closed_forms(N=37, d=5, wl=6, wr=3):
    """With Q = 0 every visible score equals the bias, so P is uniform (or geometric)."""
    r = np.random.default_rng(3)
    v = r.standard_normal((1, N, 1, d))
    k = r.standard_normal((1, N, 1, d))
    q = np.zeros((1, N, 1, d))
    worst = 0.0
    # causal: key j <= i visible; count i+1
    o, lse = oracle.attention_forward(q, k, v, 0.7, True, (-1, -1), None)
    for i in range(N):
        worst = max(worst, abs(lse[0, 0, i] - math.log(i + 1)),
                    np.max(np.abs(o[0, i, 0] - v[0, :i + 1, 0].mean(0))))
    # non-causal window (wl, wr), inclusive bounds
    o, lse = oracle.attention_forward(q, k, v, 0.7, False, (wl, wr), None)
    for i in range(N):
        lo, hi = max(0, i - wl), min(N - 1, i + wr)
        worst = max(worst, abs(lse[0, 0, i] - math.log(hi - lo + 1)),
                    np.max(np.abs(o[0, i, 0] - v[0, lo:hi + 1, 0].mean(0))))
    # causal window (wl, 0) with ALiBi slope a: weights e^{-a t}, t = 0..n_i-1
    a = 0.3
    o, lse = oracle.attention_forward(q, k, v, 0.7, True, (wl, 0), np.array([a]))
    for i in range(N):
        n = min(i, wl) + 1
        closed = math.log((1 - math.exp(-a * n)) / (1 - math.exp(-a)))
        w = np.exp(-a * np.arange(n))
        o_ref = (w[:, None] * v[0, i - np.arange(n), 0]).sum(0) / w.sum()
        worst = max(worst, abs(lse[0, 0, i] - closed), np.max(np.abs(o[0, i, 0] - o_ref)))
    return worst


def test_q0_closed_forms():
    assert check_q0_closed_forms() < 1e-12


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("m", MASKS)
def test_rows_of_p_sum_to_one(m):
    q, k, _, _ = rnd(1, 19, 1, 8, 11)
    rows = np.arange(19)
    s = oracle.logits(q[0, :, 0], k[0, :, 0], rows, 0.5, m["causal"], *m["window_size"],
                      0.2 if m["alibi"] else None)
    p, lse = oracle.softmax_rows(s)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(1) - 1)) < 1e-14
    # invisible keys get exactly zero probability
    vis = oracle.visible(rows[:, None], rows[None, :], m["causal"], *m["window_size"])
    assert np.all(p[~vis] == 0)


@pytest.mark.parametrize("m", MASKS)
def test_constant_v_gives_constant_output(m):
    q, k, _, _ = rnd(2, 23, 3, 6, 12)
    v = np.broadcast_to(np.array([0.5, -1.25, 2.0, 0.0, 3.5, -7.0]), (2, 23, 3, 6)).copy()
    o, _ = oracle.attention_forward(q, k, v, 0.4, m["causal"], m["window_size"], slopes_for(3, m["alibi"]))
    assert np.max(np.abs(o - v)) < 1e-13


def test_single_key():
    q, k, v, _ = rnd(2, 1, 3, 7, 13)
    o, lse = oracle.attention_forward(q, k, v, 0.3, False, (-1, -1), slopes_for(3, True))
    assert np.max(np.abs(o - v)) < 1e-15
    assert np.max(np.abs(lse - 0.3 * np.einsum("bnhd,bnhd->bhn", q, k))) < 1e-14


def test_causal_row_zero():
    q, k, v, _ = rnd(2, 17, 2, 5, 14)
    o, lse = oracle.attention_forward(q, k, v, 0.6, True, (-1, -1), slopes_for(2, True))
    assert np.max(np.abs(o[:, 0] - v[:, 0])) < 1e-15
    assert np.max(np.abs(lse[:, :, 0] - 0.6 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]))) < 1e-14


@pytest.mark.parametrize("m", MASKS)
def test_shift_invariance_in_k(m):
    """k_j -> k_j + c adds scale*q_i.c to every score of row i: O unchanged, LSE shifted."""
    q, k, v, _ = rnd(1, 21, 2, 4, 15)
    c = np.array([0.3, -1.1, 0.7, 2.0])
    sl = slopes_for(2, m["alibi"])
    o1, l1 = oracle.attention_forward(q, k, v, 0.8, m["causal"], m["window_size"], sl)
    o2, l2 = oracle.attention_forward(q, k + c, v, 0.8, m["causal"], m["window_size"], sl)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs((l2 - l1) - 0.8 * np.einsum("bnhd,d->bhn", q, c))) < 1e-12


def test_key_permutation_equivariance():
    q, k, v, _ = rnd(2, 16, 2, 4, 16)
    perm = np.random.default_rng(1).permutation(16)
    o1, l1 = oracle.attention_forward(q, k, v, 0.5)
    o2, l2 = oracle.attention_forward(q, k[:, perm], v[:, perm], 0.5)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


def test_default_scale_is_inverse_sqrt_d():
    q, k, v, _ = rnd(1, 9, 1, 16, 17)
    o1, l1 = oracle.attention_forward(q, k, v, None)
    o2, l2 = oracle.attention_forward(q, k, v, 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- online softmax recurrence

def check_online_softmax(N=29, seed=18):
    q, k, v, _ = rnd(1, N, 2, 6, seed)
    worst = 0.0
    for m in MASKS:
        sl = slopes_for(2, m["alibi"])
        o_ref, l_ref = oracle.attention_forward(q, k, v, 0.45, m["causal"], m["window_size"], sl)
        for block in (1, 3, 16, N):
            for deferred in (True, False):
                o, l = oracle.online_softmax_attention(q, k, v, block, 0.45, m["causal"],
                                                       m["window_size"], sl, deferred=deferred)
                worst = max(worst, np.max(np.abs(o - o_ref)), np.max(np.abs(l - l_ref)))
    return worst


def test_online_softmax_matches_definition():
    assert check_online_softmax() < 1e-12


# ---------------------------------------------------------------- library cross-check

def torch_sdpa_reference(q, k, v, scale, causal, window, slopes):
    """torch CPU float64 scaled_dot_product_attention with an explicit additive mask."""
    B, N, H, d = q.shape
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    allowed = torch.ones(N, N, dtype=torch.bool)
    wl, wr = window
    if causal:
        allowed &= j <= i
        wr = 0
    if wl >= 0:
        allowed &= j >= i - wl
    if wr >= 0:
        allowed &= j <= i + wr
    bias = torch.zeros(H, N, N, dtype=torch.float64)
    if slopes is not None:
        bias = -torch.from_numpy(slopes)[:, None, None] * (i - j).abs().double()
    bias = bias.masked_fill(~allowed, float("-inf"))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=bias[None], scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("m", MASKS)
def test_matches_torch_cpu_sdpa(m):
    q, k, v, _ = rnd(2, 33, 3, 8, 19)
    sl = slopes_for(3, m["alibi"])
    o, _ = oracle.attention_forward(q, k, v, 0.35, m["causal"], m["window_size"], sl)
    o_t = torch_sdpa_reference(q, k, v, 0.35, m["causal"], m["window_size"], sl)
    assert np.max(np.abs(o - o_t)) < 1e-12


# ---------------------------------------------------------------- gradients

def numeric_grads(q, k, v, do, scale, causal, window, sl, h=1e-6):
    def loss(qq, kk, vv):
        o, _ = oracle.attention_forward(qq, kk, vv, scale, causal, window, sl)
        return float(np.sum(o * do))
    out = []
    for which in range(3):
        arrs = [q, k, v]
        g = np.zeros_like(arrs[which])
        it = np.nditer(arrs[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in arrs]
            minus = [a.copy() for a in arrs]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        out.append(g)
    return out


@pytest.mark.parametrize("m", MASKS)
def test_backward_matches_finite_differences(m):
    q, k, v, do = rnd(1, 6, 2, 3, 20)
    sl = slopes_for(2, m["alibi"])
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.9, m["causal"], m["window_size"], sl)
    nq, nk, nv = numeric_grads(q, k, v, do, 0.9, m["causal"], m["window_size"], sl)
    assert np.max(np.abs(dq - nq)) < 1e-7
    assert np.max(np.abs(dk - nk)) < 1e-7
    assert np.max(np.abs(dv - nv)) < 1e-7


@pytest.mark.parametrize("m", MASKS)
def test_backward_matches_torch_autograd(m):
    q, k, v, do = rnd(2, 18, 2, 5, 21)
    sl = slopes_for(2, m["alibi"])
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    B, N, H, d = q.shape
    s = torch.einsum("bihd,bjhd->bhij", tq, tk) * 0.6
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    if sl is not None:
        s = s - torch.from_numpy(sl)[None, :, None, None] * (i - j).abs().double()
    vis = torch.from_numpy(oracle.visible(i.numpy(), j.numpy(), m["causal"], *m["window_size"]))
    s = s.masked_fill(~vis, float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), tv)
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.6, m["causal"], m["window_size"], sl)
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


def test_gradient_identities():
    q, k, v, do = rnd(2, 25, 2, 6, 22)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, True, (7, 0), slopes_for(2, True))
    # rows of P sum to 1, so the dV rows sum to the dO rows (every row sees itself)
    assert np.max(np.abs(dv.sum(1) - do.sum(1))) < 1e-12
    # sum_j dS_ij = 0, so dQ = 0 when every key row is the same vector
    kc = np.broadcast_to(k[:, :1], k.shape).copy()
    dq0, _, _ = oracle.attention_backward(q, kc, v, do, 0.5, True, (7, 0), slopes_for(2, True))
    assert np.max(np.abs(dq0)) < 1e-12
    # dK sums to zero over keys of a head for the same reason (sum_j dS_ij = 0)
    assert np.max(np.abs(dk.sum(1))) < 1e-12


@pytest.mark.parametrize("m", MASKS)
def test_sampled_rows_match_full(m):
    q, k, v, do = rnd(2, 40, 3, 4, 23)
    sl = slopes_for(3, m["alibi"])
    o, lse = oracle.attention_forward(q, k, v, 0.5, m["causal"], m["window_size"], sl)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, m["causal"], m["window_size"], sl)
    rows = np.array([[0, 0, 0], [1, 2, 39], [0, 1, 17], [1, 0, 5]])
    o_r, lse_r = oracle.attention_forward_rows(q, k, v, rows, 0.5, m["causal"], m["window_size"], sl)
    keys = np.array([[1, 2, 0], [0, 1, 39], [1, 2, 11]])
    dq_r, dk_r, dv_r = oracle.attention_backward_sampled(q, k, v, do, rows, keys, 0.5, m["causal"],
                                                         m["window_size"], sl)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o_r[n] - o[b, i, h])) < 1e-13
        assert abs(lse_r[n] - lse[b, h, i]) < 1e-13
        assert np.max(np.abs(dq_r[n] - dq[b, i, h])) < 1e-13
    for n, (b, h, j) in enumerate(keys):
        assert np.max(np.abs(dk_r[n] - dk[b, j, h])) < 1e-12
        assert np.max(np.abs(dv_r[n] - dv[b, j, h])) < 1e-12


def test_bf16_inputs_upcast_exactly():
    t = torch.randn(1, 5, 1, 4).to(torch.bfloat16)
    assert np.array_equal(oracle.to_f64(t), t.double().numpy())


# ---------------------------------------------------------------- planted mistakes

def _all_pins_pass():
    try:
        return (check_golden_forward() < 1e-14 and check_golden_backward() < 1e-14
                and check_q0_closed_forms() < 1e-12 and check_online_softmax(N=13) < 1e-12)
    except Exception:
        return False


MUTANTS = {}


def _mutant(name):
    def reg(f):
        MUTANTS[name] = f
        return f
    return reg


@_mutant("window_left_exclusive")
def _m1(mp):
    orig = oa.visible

    def bad(i, j, causal, wl, wr):
        ok = orig(i, j, causal, wl, wr)
        if wl >= 0:
            ok &= np.asarray(j) > np.asarray(i) - wl
        return ok
    mp.setattr(oa, "visible", bad)


@_mutant("alibi_sign_flipped")
def _m2(mp):
    orig = oa._slope
    mp.setattr(oa, "_slope", lambda s, h: None if s is None else -orig(s, h))


@_mutant("alibi_bias_scaled")
def _m3(mp):
    orig = oa.logits

    def bad(q_rows, k_head, rows, scale, causal, wl, wr, slope):
        return orig(q_rows, k_head, rows, scale, causal, wl, wr,
                    None if slope is None else slope * scale)
    mp.setattr(oa, "logits", bad)


@_mutant("lse_in_log2")
def _m4(mp):
    orig = oa.softmax_rows

    def bad(s):
        p, lse = orig(s)
        return p, lse / math.log(2)
    mp.setattr(oa, "softmax_rows", bad)


@_mutant("delta_term_dropped")
def _m5(mp):
    mp.setattr(oa, "_row_grads", lambda s, p, do, vh: (p * (do @ vh.T), np.zeros(len(p))))


@_mutant("dk_missing_scale")
def _m6(mp):
    orig = oa.attention_backward

    def bad(*a, **kw):
        dq, dk, dv = orig(*a, **kw)
        return dq, dk * 2.0, dv
    mp.setattr(oa, "attention_backward", bad)
    mp.setattr(oracle, "attention_backward", bad)


@_mutant("causal_excludes_diagonal")
def _m7(mp):
    orig = oa.visible

    def bad(i, j, causal, wl, wr):
        ok = orig(i, j, causal, wl, wr)
        if causal:
            ok &= np.asarray(j) < np.asarray(i)
        return ok
    mp.setattr(oa, "visible", bad)


@_mutant("transposed_v")
def _m8(mp):
    orig = oa.attention_forward

    def bad(q, k, v, *a, **kw):
        return orig(q, k, oa.to_f64(k), *a, **kw)
    mp.setattr(oa, "attention_forward", bad)
    mp.setattr(oracle, "attention_forward", bad)


def test_unmutated_oracle_passes_all_pins():
    assert _all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert not _all_pins_pass(), f"mistake {name} was not caught by any pin"
