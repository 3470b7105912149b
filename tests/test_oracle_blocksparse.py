"""Pins for the block-sparse oracle (128 x 128 block mask on top of the dense masks).

The reading pinned here (wmrh.cn FlashAttention v2 article, section 6, suggests
block-sparse patterns; the page fixes no format): key j is visible to query i
when the dense rule allows it and mask[b, h, i // 128, j // 128] != 0; a row
with no visible key gives O = 0, LSE = -inf and zero gradients. Checked against:
* torch CPU float64 scaled_dot_product_attention and logsumexp with an explicit
  additive mask built here element by element;
* torch autograd through the same masked formulation;
* the dense oracle (all-ones mask) and the variable-length oracle (a
  block-diagonal mask is a batch of 128-token sequences);
* planted mistakes, each caught by one of the pins.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import blocksparse as ob

MASKS = [
    dict(causal=False, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(200, 0), alibi=True),
    dict(causal=False, window_size=(90, 40), alibi=True),
]


def slopes(H, on):
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]) if on else None


def rnd(B, N, H, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, N, H, d)) for _ in range(4)]


def random_block_mask(B, H, N, seed, density=0.5, diag=True):
    nb = -(-N // 128)
    r = np.random.default_rng(seed)
    m = (r.random((B, H, nb, nb)) < density).astype(np.uint8)
    if diag:
        m[:, :, np.arange(nb), np.arange(nb)] = 1
    return m


def element_mask(block_mask_bh, N, causal, window):
    """[N, N] visibility built position by position (no block indexing tricks)."""
    allowed = np.zeros((N, N), dtype=bool)
    wl, wr = window
    if causal:
        wr = 0
    for i in range(N):
        for j in range(N):
            ok = block_mask_bh[i // 128][j // 128] != 0
            ok = ok and (not causal or j <= i) and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)
            allowed[i, j] = ok
    return allowed


def torch_masked(q, k, v, bm, scale, causal, window, sl):
    """Per (b, h): torch SDPA and logsumexp with an explicit additive mask. Rows with
    no visible key are returned as NaN rows (SDPA's result there), flagged in `empty`."""
    B, N, H, d = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    empty = np.zeros((B, H, N), dtype=bool)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    for b in range(B):
        for h in range(H):
            allowed = element_mask(bm[b, h], N, causal, window)
            bias = np.zeros((N, N)) if sl is None else -sl[h] * np.abs(i - j)
            add = torch.from_numpy(np.where(allowed, bias, -np.inf))
            tq, tk, tv = (torch.from_numpy(x[b, :, h, :].copy()) for x in (q, k, v))
            o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=add[None],
                                                                 scale=scale)[0]
            out[b, :, h, :] = o.numpy()
            lse[b, h] = torch.logsumexp(scale * tq @ tk.T + add, dim=-1).numpy()
            empty[b, h] = ~allowed.any(axis=1)
    return out, lse, empty


def check_library(m, N=300, seed=5):
    q, k, v, _ = rnd(2, N, 2, 6, seed)
    bm = random_block_mask(2, 2, N, seed + 1, density=0.4, diag=False)
    sl = slopes(2, m["alibi"])
    o, lse = ob.blocksparse_forward(q, k, v, bm, 0.4, m["causal"], m["window_size"], sl)
    o_t, lse_t, empty = torch_masked(q, k, v, bm, 0.4, m["causal"], m["window_size"], sl)
    e = ~empty
    worst = max(np.max(np.abs(o.transpose(0, 2, 1, 3)[e] - o_t.transpose(0, 2, 1, 3)[e])),
                np.max(np.abs(lse[e] - lse_t[e])))
    # rows with no visible key: O = 0, LSE = -inf
    if empty.any():
        assert np.all(o.transpose(0, 2, 1, 3)[empty] == 0.0) and np.all(lse[empty] == -np.inf)
    return worst, int(empty.sum())


@pytest.mark.parametrize("m", MASKS)
def test_matches_torch_sdpa_with_an_elementwise_mask(m):
    worst, _ = check_library(m)
    assert worst < 1e-12


def test_some_rows_have_no_visible_key_and_get_zero_output():
    _, n_empty = check_library(MASKS[1])
    assert n_empty > 0  # the random mask leaves whole causal rows empty: the convention is exercised


@pytest.mark.parametrize("m", MASKS)
def test_backward_matches_torch_autograd(m):
    B, N, H, d = 1, 260, 2, 5
    q, k, v, do = rnd(B, N, H, d, 7)
    bm = random_block_mask(B, H, N, 8, density=0.5, diag=True)  # diagonal on: no empty row
    sl = slopes(H, m["alibi"])
    dq, dk, dv = ob.blocksparse_backward(q, k, v, do, bm, 0.6, m["causal"], m["window_size"], sl)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    for h in range(H):
        allowed = torch.from_numpy(element_mask(bm[0, h], N, m["causal"], m["window_size"]))
        tq, tk, tv = (torch.from_numpy(x[0, :, h, :].copy()).requires_grad_(True) for x in (q, k, v))
        s = 0.6 * tq @ tk.T
        if sl is not None:
            s = s - sl[h] * torch.from_numpy(np.abs(i - j).astype(np.float64))
        o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=-1) @ tv
        (o * torch.from_numpy(do[0, :, h, :])).sum().backward()
        assert np.max(np.abs(dq[0, :, h] - tq.grad.numpy())) < 1e-12
        assert np.max(np.abs(dk[0, :, h] - tk.grad.numpy())) < 1e-12
        assert np.max(np.abs(dv[0, :, h] - tv.grad.numpy())) < 1e-12


def test_empty_rows_have_zero_gradients_and_do_not_leak():
    B, N, H, d = 1, 384, 1, 4
    q, k, v, do = rnd(B, N, H, d, 9)
    bm = np.ones((1, 1, 3, 3), dtype=np.uint8)
    bm[0, 0, 1, :] = 0  # query block 1 sees nothing
    dq, dk, dv = ob.blocksparse_backward(q, k, v, do, bm, 0.5, False)
    assert np.all(dq[0, 128:256] == 0.0)
    do2 = do.copy()
    do2[0, 128:256] += 5.0  # gradients flowing from empty rows must be zero
    dq2, dk2, dv2 = ob.blocksparse_backward(q, k, v, do2, bm, 0.5, False)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


@pytest.mark.parametrize("m", MASKS)
def test_all_ones_mask_is_the_dense_definition(m):
    q, k, v, do = rnd(1, 270, 2, 4, 11)
    sl = slopes(2, m["alibi"])
    bm = np.ones((1, 2, 3, 3), dtype=np.uint8)
    o, lse = ob.blocksparse_forward(q, k, v, bm, 0.5, m["causal"], m["window_size"], sl)
    o_d, lse_d = oracle.attention_forward(q, k, v, 0.5, m["causal"], m["window_size"], sl)
    assert np.array_equal(o, o_d) and np.array_equal(lse, lse_d)


def test_block_diagonal_mask_is_a_batch_of_128_token_sequences():
    B, N, H, d = 1, 384, 2, 4
    q, k, v, do = rnd(B, N, H, d, 12)
    bm = np.zeros((1, H, 3, 3), dtype=np.uint8)
    bm[0, :, np.arange(3), np.arange(3)] = 1
    o, lse = ob.blocksparse_forward(q, k, v, bm, 0.5, True)
    g = ob.blocksparse_backward(q, k, v, do, bm, 0.5, True)
    cu = [0, 128, 256, 384]
    o_v, lse_v = oracle.varlen_forward(q[0], k[0], v[0], cu, 0.5, True)
    g_v = oracle.varlen_backward(q[0], k[0], v[0], do[0], cu, 0.5, True)
    assert np.max(np.abs(o[0] - o_v)) < 1e-13 and np.max(np.abs(lse[0] - lse_v)) < 1e-13
    for a, b in zip(g, g_v):
        assert np.max(np.abs(a[0] - b)) < 1e-13


@pytest.mark.parametrize("m", MASKS)
def test_sampled_rows_match_full(m):
    q, k, v, do = rnd(2, 280, 2, 4, 13)
    bm = random_block_mask(2, 2, 280, 14, density=0.6, diag=False)
    sl = slopes(2, m["alibi"])
    o, lse = ob.blocksparse_forward(q, k, v, bm, 0.5, m["causal"], m["window_size"], sl)
    dq, dk, dv = ob.blocksparse_backward(q, k, v, do, bm, 0.5, m["causal"], m["window_size"], sl)
    rows = np.array([[0, 0, 0], [1, 1, 279], [0, 1, 130], [1, 0, 255]])
    keys = np.array([[1, 1, 0], [0, 0, 200], [1, 1, 128]])
    o_r, lse_r = ob.blocksparse_forward_rows(q, k, v, bm, rows, 0.5, m["causal"], m["window_size"], sl)
    dq_r, dk_r, dv_r = ob.blocksparse_backward_sampled(q, k, v, do, bm, rows, keys, 0.5, m["causal"],
                                                       m["window_size"], sl)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o_r[n] - o[b, i, h])) < 1e-13
        assert lse_r[n] == lse[b, h, i] or abs(lse_r[n] - lse[b, h, i]) < 1e-13
        assert np.max(np.abs(dq_r[n] - dq[b, i, h])) < 1e-13
    for n, (b, h, j) in enumerate(keys):
        assert np.max(np.abs(dk_r[n] - dk[b, j, h])) < 1e-12
        assert np.max(np.abs(dv_r[n] - dv[b, j, h])) < 1e-12


# ---------------------------------------------------------------- planted mistakes

def _all_pins_pass():
    try:
        return all(check_library(m)[0] < 1e-12 for m in MASKS)
    except Exception:
        return False


MUTANTS = {}


def _mutant(name):
    def reg(f):
        MUTANTS[name] = f
        return f
    return reg


@_mutant("mask_transposed")
def _m1(mp):
    orig = ob.key_mask_rows
    mp.setattr(ob, "key_mask_rows", lambda m, rows, N, block=128: orig(np.asarray(m).T, rows, N, block))


@_mutant("block_size_256")
def _m2(mp):
    orig = ob.key_mask_rows
    mp.setattr(ob, "key_mask_rows", lambda m, rows, N, block=128: orig(m, rows, N, 256))


@_mutant("mask_ignored")
def _m3(mp):
    mp.setattr(ob, "key_mask_rows", lambda m, rows, N, block=128: np.ones((len(rows), N), dtype=bool))


@_mutant("mask_of_wrong_head")
def _m4(mp):
    mp.setattr(ob, "_mask_of", lambda bm, b, h: np.asarray(bm)[b, (h + 1) % np.asarray(bm).shape[1]])


def test_unmutated_blocksparse_oracle_passes_all_pins():
    assert _all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_blocksparse_mistake_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert not _all_pins_pass(), f"mistake {name} was not caught by any pin"
