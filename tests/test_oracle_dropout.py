"""Pins for the dropout oracle (keep matrix from Philox4x32-10, weights rescaled by 1/(1-p)).

The reading pinned here (wmrh.cn FlashAttention v2 article, section 5.1, names
dropout_p; the page fixes no generator): O = (softmax(S) * Z) V / (1 - p), LSE
undropped, Z from Philox4x32-10 with key (seed mod 2^32, seed div 2^32) and
counter (g, i, b*H + h, offset), key j taking the 8-bit value t (bits 8*(t%4) of
word t//4) with g = 2*(j//32) + (j//8)%2 and t = 8*((j//16)%2) + j%8, kept iff
value < floor((1-p)*256 + 0.5). Checked against:
* rocRAND's Philox4x32-10 engine (tests/c/philox_ref.cpp, a host build of the
  library's header), block by block;
* a keep matrix built in the test from that library generator and the layout
  above, pushed through torch softmax with an explicit additive mask;
* torch autograd through (softmax(S) * Z) V / (1 - p) for the gradients;
* the dense oracle (p = 0, and LSE for every p), the expectation over seeds
  (the 1/(1-p) rescale), keep-rate and uniformity statistics;
* planted mistakes, each caught by one of the pins.
"""
import functools
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from oracle import dropout as od

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def rnd(B, N, H, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, N, H, d)) for _ in range(4)]


@functools.lru_cache(maxsize=None)
def _reference_program():
    """Host build of tests/c/philox_ref.cpp against rocRAND's header (cached per session)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc for the rocRAND reference generator")
    exe = os.path.join(tempfile.mkdtemp(prefix="philox_ref_"), "philox_ref")
    build = subprocess.run([hipcc, "--cuda-host-only", "-O2", "-std=c++17",
                            os.path.join(ROOT, "tests", "c", "philox_ref.cpp"), "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    return exe


def library_blocks(jobs):
    """Philox4x32-10 blocks from rocRAND's engine: jobs = [(counter[4], key[2]), ...]."""
    text = "".join(" ".join("%x" % (int(x) & 0xFFFFFFFF) for x in (*c, *k)) + "\n" for c, k in jobs)
    run = subprocess.run([_reference_program()], input=text, capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    return [[int(w, 16) for w in line.split()] for line in run.stdout.splitlines()]


def library_keep(bh, N, p, seed, offset):
    """[N, N] keep matrix of head bh built from rocRAND's Philox and the stated layout."""
    T = int(np.floor((1.0 - float(np.float32(p))) * 256.0 + 0.5))
    key = (seed & 0xFFFFFFFF, seed >> 32)
    groups = 2 * ((N + 31) // 32)
    blocks = library_blocks([((g, i, bh, offset), key) for i in range(N) for g in range(groups)])
    z = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for g in range(groups):
            w = blocks[i * groups + g]
            # group g: the keys of block g // 2 with bit 3 equal to g % 2, in increasing order
            keys = [32 * (g // 2) + 8 * (g % 2) + 16 * (t // 8) + t % 8 for t in range(16)]
            for t, j in enumerate(keys):
                if j < N:
                    z[i, j] = ((w[t // 4] >> (8 * (t % 4))) & 0xFF) < T
    return z


# ---------------------------------------------------------------- the generator

def test_philox_matches_rocrand_library():
    r = np.random.default_rng(100)
    jobs = [((0, 0, 0, 0), (0, 0)), ((2**32 - 1,) * 4, (2**32 - 1, 2**32 - 1))]
    jobs += [(tuple(int(x) for x in r.integers(0, 2**32, 4)), tuple(int(x) for x in r.integers(0, 2**32, 2)))
             for _ in range(30)]
    ref = library_blocks(jobs)
    for (c, k), want in zip(jobs, ref):
        assert [int(x) for x in od.philox4x32(np.array(c, dtype=np.uint64), k)] == want


def test_philox_vectorised_over_counters():
    key = (0x01234567, 0x89ABCDEF)
    ctrs = np.array([[g, i, 5, 9] for i in range(3) for g in range(4)], dtype=np.uint64)
    out = od.philox4x32(ctrs, key)
    ref = library_blocks([([int(x) for x in c], key) for c in ctrs])
    for n in range(len(ctrs)):
        assert [int(x) for x in out[n]] == ref[n]


def test_value_layout_matches_library_blocks():
    seed, offset, bh, N = 0x1234_0000_5678, 7, 3, 70
    vals = od.random_values(bh, np.arange(5), N, seed, offset)
    ref = library_blocks([((2 * (j // 32) + (j // 8) % 2, i, bh, offset), (0x5678, 0x1234))
                          for i in range(5) for j in range(N)])
    for i in range(5):
        for j in range(N):
            w, t = ref[i * N + j], 8 * ((j // 16) % 2) + j % 8
            assert vals[i, j] == (w[t // 4] >> (8 * (t % 4))) & 0xFF
    # each group's sixteen values are used once: its keys are a partition of the block
    for i in range(5):
        for g in range(4):
            got = sorted(int(vals[i, j]) for j in range(N) if 2 * (j // 32) + (j // 8) % 2 == g)
            w = ref[i * N + (32 * (g // 2) + 8 * (g % 2))]
            assert got == sorted((w[t // 4] >> (8 * (t % 4))) & 0xFF for t in range(16))


def test_offset_is_a_32_bit_counter_word():
    od.random_values(0, [0], 16, 1, 2**32 - 1)
    for bad in (2**32, -1):
        with pytest.raises(ValueError):
            od.random_values(0, [0], 16, 1, bad)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate_matches_threshold(p):
    z = od.keep_rows(11, np.arange(512), 512, p, seed=99, offset=0)
    n = z.size
    q = od.keep_threshold(p) / 256.0
    assert abs(q - (1 - p)) <= 2.0 ** -9
    assert abs(z.mean() - q) < 6 * np.sqrt(q * (1 - q) / n)


def test_values_are_uniform_and_heads_independent():
    v = od.random_values(0, np.arange(256), 4096, seed=5, offset=1)
    assert v.max() <= 255
    hist = np.bincount(v.ravel(), minlength=256)
    e = v.size / 256
    chi2 = float(((hist - e) ** 2 / e).sum())
    assert chi2 < 256 + 8 * np.sqrt(2 * 256)
    z0 = od.keep_rows(0, np.arange(256), 256, 0.5, 5, 1).astype(float)
    z1 = od.keep_rows(1, np.arange(256), 256, 0.5, 5, 1).astype(float)
    z2 = od.keep_rows(0, np.arange(256), 256, 0.5, 5, 2).astype(float)
    for other in (z1, z2, z0.T):
        c = np.corrcoef(z0.ravel(), other.ravel())[0, 1]
        assert abs(c) < 6 / np.sqrt(z0.size)


def test_p_zero_keeps_everything():
    assert od.keep_threshold(0.0) == 256
    assert od.keep_threshold(0.999) == 0 and not od.keep_rows(0, np.arange(64), 64, 0.999, 1, 2).any()
    assert od.keep_rows(0, np.arange(64), 64, 0.0, 1, 2).all()
    with pytest.raises(ValueError):
        od.keep_threshold(1.0)
    with pytest.raises(ValueError):
        od.keep_threshold(-0.1)


# ---------------------------------------------------------------- forward

MASKS = [
    dict(causal=False, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(-1, -1), alibi=False),
    dict(causal=True, window_size=(20, 0), alibi=True),
    dict(causal=False, window_size=(9, 13), alibi=True),
]


def slopes(H, on):
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]) if on else None


def torch_with_mask(q, k, v, m, p, seed, offset, scale):
    """(softmax(S) * Z) V / (1 - p) in torch fp64 with an explicit additive mask and Z from rocRAND's Philox."""
    B, N, H, d = q.shape
    sl = slopes(H, m["alibi"])
    out = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    wl, wr = m["window_size"]
    if m["causal"]:
        wr = 0
    allowed = (wl < 0) | (j >= i - wl)
    allowed &= (wr < 0) | (j <= i + wr)
    for b in range(B):
        for h in range(H):
            bias = np.zeros((N, N)) if sl is None else -sl[h] * np.abs(i - j)
            add = torch.from_numpy(np.where(allowed, bias, -np.inf))
            tq, tk, tv = (torch.from_numpy(x[b, :, h, :].copy()) for x in (q, k, v))
            s = scale * tq @ tk.T + add
            pt = torch.softmax(s, dim=-1)
            z = torch.from_numpy(library_keep(b * H + h, N, p, seed, offset).astype(np.float64))
            out[b, :, h, :] = ((pt * z) @ tv / (1 - float(np.float32(p)))).numpy()
            lse[b, h] = torch.logsumexp(s, dim=-1).numpy()
    return out, lse


def check_forward(m, p=0.3, seed=21, offset=4):
    q, k, v, _ = rnd(2, 37, 2, 5, 31)
    o, lse = od.dropout_forward(q, k, v, p, seed, offset, 0.45, m["causal"], m["window_size"],
                                slopes(2, m["alibi"]))
    o_t, lse_t = torch_with_mask(q, k, v, m, p, seed, offset, 0.45)
    return max(np.max(np.abs(o - o_t)), np.max(np.abs(lse - lse_t)))


@pytest.mark.parametrize("m", MASKS)
def test_forward_matches_torch_with_library_keep_matrix(m):
    assert check_forward(m) < 1e-12


@pytest.mark.parametrize("m", MASKS)
def test_p_zero_is_the_dense_definition_and_lse_is_undropped(m):
    q, k, v, _ = rnd(1, 50, 2, 4, 3)
    sl = slopes(2, m["alibi"])
    o0, lse0 = od.dropout_forward(q, k, v, 0.0, 8, 0, 0.5, m["causal"], m["window_size"], sl)
    o_d, lse_d = oracle.attention_forward(q, k, v, 0.5, m["causal"], m["window_size"], sl)
    assert np.array_equal(o0, o_d) and np.array_equal(lse0, lse_d)
    _, lse1 = od.dropout_forward(q, k, v, 0.4, 8, 0, 0.5, m["causal"], m["window_size"], sl)
    assert np.array_equal(lse1, lse_d)


def test_expectation_over_seeds_is_the_undropped_output():
    q, k, v, _ = rnd(1, 12, 1, 3, 4)
    o_d, _ = oracle.attention_forward(q, k, v, 0.6, True)
    samples = np.stack([od.dropout_forward(q, k, v, 0.5, s, 0, 0.6, True)[0] for s in range(1500)])
    mean, sem = samples.mean(0), samples.std(0) / np.sqrt(len(samples))
    assert np.all(np.abs(mean - o_d) <= 6 * sem + 1e-12)


def test_rows_without_visible_keys_cannot_occur_and_masked_keys_stay_zero():
    # window (0, 0): each query sees only itself; O_i = z_ii * v_i / (1 - p)
    q, k, v, _ = rnd(1, 40, 1, 3, 5)
    o, lse = od.dropout_forward(q, k, v, 0.5, 77, 0, 0.5, False, (0, 0))
    z = od.keep_rows(0, np.arange(40), 40, 0.5, 77, 0)
    expect = np.where(np.diag(z)[:, None], v[0, :, 0, :] * 2.0, 0.0)
    assert np.max(np.abs(o[0, :, 0, :] - expect)) < 1e-12
    assert np.allclose(lse[0, 0], 0.5 * np.sum(q[0, :, 0, :] * k[0, :, 0, :], axis=1), atol=1e-12)


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("m", MASKS)
def test_backward_matches_torch_autograd(m):
    B, N, H, d = 1, 33, 2, 4
    q, k, v, do = rnd(B, N, H, d, 41)
    p, seed, offset = 0.25, 17, 3
    sl = slopes(H, m["alibi"])
    dq, dk, dv = od.dropout_backward(q, k, v, do, p, seed, offset, 0.6, m["causal"], m["window_size"], sl)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    wl, wr = m["window_size"]
    if m["causal"]:
        wr = 0
    allowed = torch.from_numpy(((wl < 0) | (j >= i - wl)) & ((wr < 0) | (j <= i + wr)))
    for h in range(H):
        tq, tk, tv = (torch.from_numpy(x[0, :, h, :].copy()).requires_grad_(True) for x in (q, k, v))
        s = 0.6 * tq @ tk.T
        if sl is not None:
            s = s - sl[h] * torch.from_numpy(np.abs(i - j).astype(np.float64))
        z = torch.from_numpy(library_keep(h, N, p, seed, offset).astype(np.float64))
        o = (torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=-1) * z) @ tv / (1 - float(np.float32(p)))
        (o * torch.from_numpy(do[0, :, h, :])).sum().backward()
        assert np.max(np.abs(dq[0, :, h] - tq.grad.numpy())) < 1e-12
        assert np.max(np.abs(dk[0, :, h] - tk.grad.numpy())) < 1e-12
        assert np.max(np.abs(dv[0, :, h] - tv.grad.numpy())) < 1e-12


def test_backward_at_p_zero_is_the_dense_backward():
    q, k, v, do = rnd(1, 30, 2, 4, 6)
    g = od.dropout_backward(q, k, v, do, 0.0, 1, 0, 0.5, True)
    g_d = oracle.attention_backward(q, k, v, do, 0.5, True)
    for a, b in zip(g, g_d):
        assert np.max(np.abs(a - b)) < 1e-13


@pytest.mark.parametrize("m", MASKS[1:3])
def test_sampled_rows_match_full(m):
    q, k, v, do = rnd(2, 45, 2, 4, 13)
    sl = slopes(2, m["alibi"])
    args = (0.2, 5, 9, 0.5, m["causal"], m["window_size"], sl)
    o, lse = od.dropout_forward(q, k, v, *args)
    dq, dk, dv = od.dropout_backward(q, k, v, do, *args)
    rows = np.array([[0, 0, 0], [1, 1, 44], [0, 1, 17], [1, 0, 31]])
    keys = np.array([[1, 1, 0], [0, 0, 40], [1, 1, 16]])
    o_r, lse_r = od.dropout_forward_rows(q, k, v, rows, *args)
    dq_r, dk_r, dv_r = od.dropout_backward_sampled(q, k, v, do, rows, keys, *args)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o_r[n] - o[b, i, h])) < 1e-13
        assert abs(lse_r[n] - lse[b, h, i]) < 1e-13
        assert np.max(np.abs(dq_r[n] - dq[b, i, h])) < 1e-13
    for n, (b, h, j) in enumerate(keys):
        assert np.max(np.abs(dk_r[n] - dk[b, j, h])) < 1e-12
        assert np.max(np.abs(dv_r[n] - dv[b, j, h])) < 1e-12


# ---------------------------------------------------------------- planted mistakes

def _grad_pin():
    try:
        test_backward_matches_torch_autograd(MASKS[2])
        return True
    except AssertionError:
        return False


def _all_pins_pass():
    try:
        fwd = all(check_forward(m) < 1e-12 for m in MASKS)
        test_expectation_over_seeds_is_the_undropped_output()
        test_p_zero_is_the_dense_definition_and_lse_is_undropped(MASKS[1])
        return fwd and _grad_pin()
    except (AssertionError, ValueError):
        return False


MUTANTS = {}


def _mutant(name):
    def reg(f):
        MUTANTS[name] = f
        return f
    return reg


@_mutant("keep_matrix_transposed")
def _m1(mp):
    orig = od.keep_rows
    def f(bh, rows, N, p, seed, offset):
        full = orig(bh, np.arange(N), N, p, seed, offset)
        return full.T[np.asarray(rows)]
    mp.setattr(od, "keep_rows", f)


@_mutant("bytes_in_reverse_order")
def _m2(mp):
    orig = od.random_values
    def f(bh, rows, N, seed, offset):
        n32 = (N + 31) // 32 * 32
        v = orig(bh, rows, n32, seed, offset).reshape(len(rows), -1, 32)[:, :, ::-1]
        return v.reshape(len(rows), -1)[:, :N]
    mp.setattr(od, "random_values", f)


@_mutant("consecutive_key_groups")
def _m2b(mp):
    def f(bh, rows, N, seed, offset):
        key, c3 = od.generator_key_counter_word(seed, offset)
        j = np.arange(N)
        ctr = np.zeros((len(rows), (N + 15) // 16, 4), dtype=np.uint64)
        ctr[..., 0] = np.arange((N + 15) // 16)[None, :]
        ctr[..., 1] = np.asarray(rows)[:, None]
        ctr[..., 2], ctr[..., 3] = bh, c3
        w = od.philox4x32(ctr, key)
        t = j % 16
        return ((w[:, j // 16, t // 4] >> (8 * (t % 4)).astype(np.uint64)) & 0xFF).astype(np.uint32)
    mp.setattr(od, "random_values", f)


@_mutant("no_rescale")
def _m3(mp):
    mp.setattr(od, "_scale_of", lambda p: 1.0)


@_mutant("head_index_ignored")
def _m4(mp):
    orig = od.keep_rows
    mp.setattr(od, "keep_rows", lambda bh, rows, N, p, seed, offset: orig(0, rows, N, p, seed, offset))


@_mutant("lse_of_dropped_weights")
def _m5(mp):
    orig = od.dropout_forward
    def f(q, k, v, p, seed, offset=0, *a, **kw):
        o, lse = orig(q, k, v, p, seed, offset, *a, **kw)
        return o, lse + np.log1p(-float(np.float32(p)))
    mp.setattr(od, "dropout_forward", f)


@_mutant("ds_without_keep_matrix")
def _m6(mp):
    mp.setattr(od, "_dropout_row_grads",
               lambda p, z, rp, do, o, vh: p * ((do @ vh.T) - np.sum(do * o, axis=1, keepdims=True)))


@_mutant("threshold_off_by_half")
def _m7(mp):
    mp.setattr(od, "keep_threshold", lambda p: int(np.floor((1.0 - float(np.float32(p))) * 128.0 + 0.5)))


def test_unmutated_dropout_oracle_passes_all_pins():
    assert _all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_dropout_mistake_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert not _all_pins_pass(), f"mistake {name} was not caught by any pin"
