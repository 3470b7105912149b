"""Pins for the variable-length oracle (packed sequences with cu_seqlens).

The reading pinned here: every packed sequence is its own attention problem,
positions count from its first token, and the logsumexp is stored [H, T]
(wmrh.cn FlashAttention v2 article, section 6, names variable-length batches;
the page fixes no interface). Checked against:
* torch CPU float64 scaled_dot_product_attention over the whole packed batch
  with a block-diagonal additive mask built here (a library routine and a
  different formulation: one big masked problem instead of slices);
* torch autograd through the same block-diagonal formulation;
* the closed form Q = 0 (LSE = ln of the number of visible keys, counted from
  the sequence's own start);
* invariance of a sequence's outputs to the contents of the others;
* planted mistakes in the slicing, each caught by one of the pins.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import varlen as ov
import workloads

MASKS = [
    dict(causal=False, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(3, 0), alibi=True),
    dict(causal=False, window_size=(2, 4), alibi=True),
]

CU_CASES = [
    [0, 5, 12, 13, 30],        # ragged, a length-1 sequence
    [0, 0, 9, 9, 21, 21],      # empty sequences in between and at the end
    [0, 17],                   # one sequence
]


def slopes(H, on):
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]) if on else None


def packed(T, H, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((T, H, d)) for _ in range(4)]


def block_diag_bias(cu, T, H, causal, window, sl):
    """[H, T, T] additive mask: -inf across sequences and outside the mask; ALiBi inside."""
    seq = np.zeros(T, dtype=np.int64)
    start = np.zeros(T, dtype=np.int64)
    for b in range(len(cu) - 1):
        seq[cu[b]:cu[b + 1]] = b
        start[cu[b]:cu[b + 1]] = cu[b]
    pos = np.arange(T) - start
    i, j = pos[:, None], pos[None, :]
    allowed = seq[:, None] == seq[None, :]
    wl, wr = window
    if causal:
        allowed &= j <= i
        wr = 0
    if wl >= 0:
        allowed &= j >= i - wl
    if wr >= 0:
        allowed &= j <= i + wr
    bias = np.zeros((H, T, T))
    if sl is not None:
        bias = -sl[:, None, None] * np.abs(i - j)[None].astype(np.float64)
    return torch.from_numpy(np.where(allowed[None], bias, -np.inf))


def torch_block_diag(q, k, v, do, cu, scale, causal, window, sl, grads=False):
    T, H, d = q.shape
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(grads) for a in (q, k, v))
    bias = block_diag_bias(cu, T, H, causal, window, sl)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2)[None], tk.permute(1, 0, 2)[None], tv.permute(1, 0, 2)[None], attn_mask=bias[None],
        scale=scale)[0].permute(1, 0, 2)
    if not grads:
        return o.detach().numpy()
    (o * torch.from_numpy(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def check_block_diag(cu, m, seed=3):
    T = cu[-1]
    q, k, v, _ = packed(T, 2, 6, seed)
    sl = slopes(2, m["alibi"])
    o, lse = oracle.varlen_forward(q, k, v, cu, 0.4, m["causal"], m["window_size"], sl)
    o_t = torch_block_diag(q, k, v, None, cu, 0.4, m["causal"], m["window_size"], sl)
    # logsumexp of the biased, masked logits of the packed batch, [H, T]
    s = 0.4 * torch.einsum("ihd,jhd->hij", torch.from_numpy(q), torch.from_numpy(k))
    lse_t = torch.logsumexp(s + block_diag_bias(cu, T, 2, m["causal"], m["window_size"], sl), dim=-1).numpy()
    return max(np.max(np.abs(o - o_t)), np.max(np.abs(lse - lse_t))) if T else 0.0


def check_q0(cu=(0, 7, 7, 20, 31), wl=4, H=2):
    """Q = 0: every visible key has the same score 0, so LSE = ln(count) with the
    count taken from the sequence's own start, and O is the mean of those V rows."""
    cu = list(cu)
    T = cu[-1]
    _, k, v, _ = packed(T, H, 3, 5)
    q = np.zeros_like(k)
    o, lse = oracle.varlen_forward(q, k, v, cu, 1.0, True, (wl, -1), None)
    worst = 0.0
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            i = t - cu[b]
            lo = cu[b] + max(0, i - wl)
            for h in range(H):
                worst = max(worst, abs(lse[h, t] - np.log(t - lo + 1)),
                            np.max(np.abs(o[t, h] - v[lo:t + 1, h].mean(0))))
    return worst


@pytest.mark.parametrize("cu", CU_CASES)
@pytest.mark.parametrize("m", MASKS)
def test_matches_block_diagonal_sdpa(cu, m):
    assert check_block_diag(cu, m) < 1e-12


def test_q0_closed_form_counts_from_each_sequence_start():
    assert check_q0() < 1e-13


@pytest.mark.parametrize("m", MASKS)
def test_backward_matches_block_diagonal_autograd(m):
    cu = [0, 4, 11, 11, 19]
    q, k, v, do = packed(19, 2, 5, 8)
    sl = slopes(2, m["alibi"])
    _, gq, gk, gv = torch_block_diag(q, k, v, do, cu, 0.7, m["causal"], m["window_size"], sl, grads=True)
    dq, dk, dv = oracle.varlen_backward(q, k, v, do, cu, 0.7, m["causal"], m["window_size"], sl)
    assert np.max(np.abs(dq - gq)) < 1e-12
    assert np.max(np.abs(dk - gk)) < 1e-12
    assert np.max(np.abs(dv - gv)) < 1e-12


def test_sequences_do_not_see_each_other():
    cu = [0, 9, 20, 26]
    q, k, v, do = packed(26, 2, 4, 9)
    o, lse = oracle.varlen_forward(q, k, v, cu, 0.5, True)
    g = oracle.varlen_backward(q, k, v, do, cu, 0.5, True)
    q2, k2, v2, do2 = (a.copy() for a in (q, k, v, do))
    for a in (q2, k2, v2, do2):
        a[9:20] += 3.0  # change only the middle sequence
    o2, lse2 = oracle.varlen_forward(q2, k2, v2, cu, 0.5, True)
    g2 = oracle.varlen_backward(q2, k2, v2, do2, cu, 0.5, True)
    keep = np.r_[0:9, 20:26]
    assert np.array_equal(o[keep], o2[keep]) and np.array_equal(lse[:, keep], lse2[:, keep])
    for x, y in zip(g, g2):
        assert np.array_equal(x[keep], y[keep])
    assert not np.allclose(o[9:20], o2[9:20])


def test_equal_lengths_match_the_fixed_length_batch():
    B, N, H, d = 3, 11, 2, 4
    r = np.random.default_rng(10)
    q, k, v, do = (r.standard_normal((B, N, H, d)) for _ in range(4))
    cu = [0, 11, 22, 33]
    o, lse = oracle.attention_forward(q, k, v, 0.5, True, (5, 0), slopes(H, True))
    ov_, lsev = oracle.varlen_forward(q.reshape(B * N, H, d), k.reshape(B * N, H, d), v.reshape(B * N, H, d), cu,
                                      0.5, True, (5, 0), slopes(H, True))
    assert np.max(np.abs(ov_ - o.reshape(B * N, H, d))) == 0.0
    assert np.max(np.abs(lsev - lse.transpose(1, 0, 2).reshape(H, B * N))) == 0.0


@pytest.mark.parametrize("m", MASKS)
def test_sampled_rows_match_full(m):
    cu = [0, 6, 6, 19, 40]
    q, k, v, do = packed(40, 3, 4, 11)
    sl = slopes(3, m["alibi"])
    o, lse = oracle.varlen_forward(q, k, v, cu, 0.5, m["causal"], m["window_size"], sl)
    dq, dk, dv = oracle.varlen_backward(q, k, v, do, cu, 0.5, m["causal"], m["window_size"], sl)
    rows = np.array([[0, 0], [2, 39], [1, 6], [0, 18], [2, 5]])
    keys = np.array([[1, 0], [0, 19], [2, 7], [2, 39]])
    o_r, lse_r = oracle.varlen_forward_rows(q, k, v, cu, rows, 0.5, m["causal"], m["window_size"], sl)
    dq_r, dk_r, dv_r = oracle.varlen_backward_sampled(q, k, v, do, cu, rows, keys, 0.5, m["causal"],
                                                      m["window_size"], sl)
    for n, (h, t) in enumerate(rows):
        assert np.max(np.abs(o_r[n] - o[t, h])) < 1e-13
        assert abs(lse_r[n] - lse[h, t]) < 1e-13
        assert np.max(np.abs(dq_r[n] - dq[t, h])) < 1e-13
    for n, (h, t) in enumerate(keys):
        assert np.max(np.abs(dk_r[n] - dk[t, h])) < 1e-12
        assert np.max(np.abs(dv_r[n] - dv[t, h])) < 1e-12


def test_varlen_workload_recipe():
    for w in workloads.VARLEN_WORKLOADS.values():
        lens = workloads.varlen_lengths(w.total, w.nseq, w.number)
        assert len(lens) == w.nseq and lens.sum() == w.total and lens.min() >= 1
        cu = workloads.cu_seqlens_from_lengths(lens)
        assert cu.dtype == torch.int32 and int(cu[0]) == 0 and int(cu[-1]) == w.total
        assert np.all(np.diff(cu.numpy()) == lens)
    t = workloads.make_varlen_inputs(50, 2, 8, "bf16", seed=4, with_dout=True)
    full = workloads.make_inputs(1, 2, 50, 8, "bf16", seed=4, with_dout=True)
    assert torch.equal(t["q"], full["q"][0]) and torch.equal(t["dout"], full["dout"][0])
    rows = workloads.sample_varlen_rows(100, 3, count=40, seed=1)
    assert len({tuple(r) for r in rows}) == 40 and rows[:, 0].max() < 3 and rows[:, 1].max() < 100


# ---------------------------------------------------------------- planted mistakes

def _all_pins_pass():
    try:
        return (all(check_block_diag(cu, m) < 1e-12 for cu in CU_CASES for m in MASKS)
                and check_q0() < 1e-13)
    except Exception:
        return False


MUTANTS = {}


def _mutant(name):
    def reg(f):
        MUTANTS[name] = f
        return f
    return reg


@_mutant("sequence_end_inclusive")
def _m1(mp):
    orig = ov.sequence_bounds
    mp.setattr(ov, "sequence_bounds", lambda cu: [(a, min(e + 1, int(cu[-1]))) for a, e in orig(cu)])


@_mutant("one_sequence_for_all")
def _m2(mp):
    mp.setattr(ov, "sequence_bounds", lambda cu: [(0, int(cu[-1]))])


@_mutant("positions_from_batch_start")
def _m3(mp):
    # slices start at token 0, so the causal/window positions of later sequences shift
    orig = ov.sequence_bounds
    mp.setattr(ov, "sequence_bounds", lambda cu: [(0, e) for _, e in orig(cu)][::-1])


@_mutant("lse_token_major")
def _m4(mp):
    orig = ov.varlen_forward

    def bad(*a, **kw):
        o, lse = orig(*a, **kw)
        return o, lse.T.reshape(lse.shape)
    mp.setattr(ov, "varlen_forward", bad)
    mp.setattr(oracle, "varlen_forward", bad)


def test_unmutated_varlen_oracle_passes_all_pins():
    assert _all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_varlen_mistake_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert not _all_pins_pass(), f"mistake {name} was not caught by any pin"
