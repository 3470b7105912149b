"""fp64 CPU oracle for attention with dropout on the attention weights — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP library and its binding never do.

Source: the wmrh.cn FlashAttention v2 article, section 5.1 (API), lists a
`dropout_p` argument next to the ones the dense oracle covers; the page fixes no
random-number generator and no formula. The plainest reading, stated here and in
the design notes:

  * Dropout acts on the normalised attention weights: with P = softmax(S) (the
    dense definition, masks and ALiBi included) and a keep matrix Z of 0/1
    entries, O = (P * Z) V / (1 - p). Each weight is kept with probability
    1 - p and the survivors are scaled so that E[O] is the undropped output.
  * The saved statistic is unchanged: LSE is that of the undropped softmax.
  * Z comes from a counter-based generator, so the backward can regenerate it:
    Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
    easy as 1, 2, 3", SC 2011), with
      key     = (seed mod 2^32, seed div 2^32)              two 32-bit words
      counter = (g, i, b * H + h, offset)                   four 32-bit words
    so offset must be below 2^32. The four 32-bit output words give sixteen
    8-bit values, the output's bytes in little-endian order (value t: bits
    8 * (t % 4) .. +7 of word t // 4). Group g holds sixteen keys of the 32-key
    block c = j // 32: g = 2c for the keys with j % 16 < 8, g = 2c + 1 for the
    others, each group's keys taking values 0 .. 15 in increasing order; i.e.
    key j takes value t = 8 * ((j // 16) % 2) + j % 8 of group
    g = 2 * (j // 32) + (j // 8) % 2. (The split matches the key halves that
    one lane half of the kernels holds.)
  * Keep iff that value < T, T = floor((1 - p) * 256 + 0.5) computed in fp64
    from the fp32 value of p. So the keep probability is T / 256: p is resolved
    to 1/256 (p = 0 keeps all), and the survivors are still scaled by 1 / (1 - p).
  * Gradients by the chain rule: dV = (P * Z)^T dO / (1 - p);
    dP = Z * (dO V^T) / (1 - p); D = rowsum(P * dP) = rowsum(dO * O);
    dS = P * (dP - D); dQ = scale * dS K; dK = scale * dS^T Q.
"""
from __future__ import annotations

import numpy as np

from . import attention as oa

# Philox4x32 round constants (the SC 2011 paper's multipliers and Weyl increments).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10
KEYS_PER_CALL = 16  # sixteen 8-bit values per call
VALUE_BITS = 8

_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32(counter, key, rounds=ROUNDS):
    """Philox4x32-R on arrays of 32-bit words (held in uint64). counter: [..., 4];
    key: (k0, k1). Each round multiplies counter words 0 and 2 by the two constants
    into 64-bit products and mixes their halves with words 1 and 3 and the key; the
    key advances by the Weyl increments between rounds. Returns [..., 4]."""
    c = [np.array(counter, dtype=np.uint64)[..., n] & _M32 for n in range(4)]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(rounds):
        if r:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0, p1 = m0 * c[0], m1 * c[2]  # below 2^64: no wrap
        c = [(p1 >> _S32) ^ c[1] ^ np.uint64(k0), p1 & _M32, (p0 >> _S32) ^ c[3] ^ np.uint64(k1), p0 & _M32]
    return np.stack(c, axis=-1)


def keep_threshold(dropout_p):
    """T: an 8-bit value v keeps its weight iff v < T."""
    p = float(np.float32(dropout_p))
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout_p must be in [0, 1)")
    return int(np.floor((1.0 - p) * 256.0 + 0.5))


def generator_key_counter_word(seed, offset):
    """(key, fourth counter word) of the stated layout; offset must be below 2^32."""
    seed, offset = int(seed), int(offset)
    if not 0 <= offset < 2 ** 32:
        raise ValueError("offset must be in [0, 2^32)")
    return (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF), offset


def random_values(bh, rows, N, seed, offset):
    """uint32 [len(rows), N]: the 8-bit value of every (query row, key) of head bh."""
    key, c3 = generator_key_counter_word(seed, offset)
    rows = np.asarray(rows, dtype=np.uint64)
    j = np.arange(N)
    g = 2 * (j // 32) + (j // 8) % 2                               # group of key j
    t = 8 * ((j // 16) % 2) + j % 8                                # its value within the group
    groups = np.arange(int(g.max()) + 1 if N else 0, dtype=np.uint64)
    ctr = np.zeros((len(rows), len(groups), 4), dtype=np.uint64)
    ctr[..., 0] = groups[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = np.uint64(bh)
    ctr[..., 3] = np.uint64(c3)
    words = philox4x32(ctr, key)                                   # [rows, groups, 4]
    vals = (words[:, g, t // 4] >> (np.uint64(VALUE_BITS) * (t % 4).astype(np.uint64))) & np.uint64(0xFF)
    return vals.astype(np.uint32)


def keep_rows(bh, rows, N, dropout_p, seed, offset):
    """Boolean Z [len(rows), N] for head bh (= b * H + h)."""
    return random_values(bh, rows, N, seed, offset) < keep_threshold(dropout_p)


def _scale_of(dropout_p):
    return 1.0 / (1.0 - float(np.float32(dropout_p)))


def dropout_forward(q, k, v, dropout_p, seed, offset=0, softmax_scale=None, causal=False,
                    window_size=(-1, -1), alibi_slopes=None):
    """q, k, v: [B, N, H, d]. Returns (out [B, N, H, d], lse [B, H, N]); lse is undropped."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    B, N, H, _ = q.shape
    rp = _scale_of(dropout_p)
    out = np.zeros((B, N, H, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, :, h, :], v[b, :, h, :]
            for r0 in range(0, N, oa.ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + oa.ROW_CHUNK))
                s = oa.logits(q[b, rows, h, :], kh, rows, scale, causal, wl, wr, oa._slope(slopes, h))
                p, lse_rows = oa.softmax_rows(s)
                z = keep_rows(b * H + h, rows, N, dropout_p, seed, offset)
                out[b, rows, h, :] = ((p * z) @ vh) * rp
                lse[b, h, rows] = lse_rows
    return out, lse


def _dropout_row_grads(p, z, rp, do_rows, o_rows, vh):
    """dP = Z * (dO V^T) / (1 - p), D = rowsum(dO * O), dS = P * (dP - D)."""
    dp = (do_rows @ vh.T) * z * rp
    dvec = np.sum(do_rows * o_rows, axis=1, keepdims=True)
    return p * (dp - dvec)


def dropout_backward(q, k, v, dout, dropout_p, seed, offset=0, softmax_scale=None, causal=False,
                     window_size=(-1, -1), alibi_slopes=None):
    """Gradients of sum(out * dout) with the same keep matrix as the forward. Returns (dq, dk, dv)."""
    out, _ = dropout_forward(q, k, v, dropout_p, seed, offset, softmax_scale, causal, window_size, alibi_slopes)
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    do = oa.to_f64(dout)
    B, N, H, _ = q.shape
    rp = _scale_of(dropout_p)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
            for r0 in range(0, N, oa.ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + oa.ROW_CHUNK))
                s = oa.logits(qh[rows], kh, rows, scale, causal, wl, wr, oa._slope(slopes, h))
                p, _ = oa.softmax_rows(s)
                z = keep_rows(b * H + h, rows, N, dropout_p, seed, offset)
                ds = _dropout_row_grads(p, z, rp, doh[rows], out[b, rows, h, :], vh)
                dv[b, :, h, :] += ((p * z) * rp).T @ doh[rows]
                dq[b, rows, h, :] = scale * (ds @ kh)
                dk[b, :, h, :] += scale * (ds.T @ qh[rows])
    return dq, dk, dv


def dropout_forward_rows(q, k, v, rows_bhi, dropout_p, seed, offset=0, softmax_scale=None, causal=False,
                         window_size=(-1, -1), alibi_slopes=None):
    """The forward at sampled (b, h, i) rows. Returns (out [n, d], lse [n])."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    B, N, H, _ = q.shape
    rp = _scale_of(dropout_p)
    rows_bhi = np.asarray(rows_bhi)
    out = np.zeros((len(rows_bhi), v.shape[-1]))
    lse = np.zeros(len(rows_bhi))
    for n, (b, h, i) in enumerate(rows_bhi):
        s = oa.logits(q[b, i, h, :][None, :], k[b, :, h, :], np.array([i]), scale, causal, wl, wr,
                      oa._slope(slopes, h))
        p, l = oa.softmax_rows(s)
        z = keep_rows(b * H + h, [i], N, dropout_p, seed, offset)
        out[n] = (((p * z) @ v[b, :, h, :]) * rp)[0]
        lse[n] = l[0]
    return out, lse


def dropout_backward_sampled(q, k, v, dout, q_rows_bhi, k_rows_bhj, dropout_p, seed, offset=0,
                             softmax_scale=None, causal=False, window_size=(-1, -1), alibi_slopes=None):
    """The backward at sampled query rows (dQ) and key rows (dK, dV). Returns (dq_rows, dk_rows, dv_rows)."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    do = oa.to_f64(dout)
    B, N, H, _ = q.shape
    rp = _scale_of(dropout_p)
    q_rows_bhi, k_rows_bhj = np.asarray(q_rows_bhi), np.asarray(k_rows_bhj)

    def head_rows(b, h, rows):
        qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
        s = oa.logits(qh[rows], kh, rows, scale, causal, wl, wr, oa._slope(slopes, h))
        p, _ = oa.softmax_rows(s)
        z = keep_rows(b * H + h, rows, N, dropout_p, seed, offset)
        o_rows = ((p * z) @ vh) * rp
        return p, z, _dropout_row_grads(p, z, rp, doh[rows], o_rows, vh)

    dq_rows = np.zeros((len(q_rows_bhi), q.shape[-1]))
    for n, (b, h, i) in enumerate(q_rows_bhi):
        _, _, ds = head_rows(b, h, np.array([i]))
        dq_rows[n] = scale * (ds @ k[b, :, h, :])[0]
    dk_rows = np.zeros((len(k_rows_bhj), k.shape[-1]))
    dv_rows = np.zeros((len(k_rows_bhj), v.shape[-1]))
    for (b, h) in sorted({(int(b), int(h)) for b, h, _ in k_rows_bhj}):
        sel = np.nonzero((k_rows_bhj[:, 0] == b) & (k_rows_bhj[:, 1] == h))[0]
        js = k_rows_bhj[sel, 2]
        for r0 in range(0, N, oa.ROW_CHUNK):
            rows = np.arange(r0, min(N, r0 + oa.ROW_CHUNK))
            p, z, ds = head_rows(b, h, rows)
            dv_rows[sel] += ((p[:, js] * z[:, js]) * rp).T @ do[b, rows, h, :]
            dk_rows[sel] += scale * (ds[:, js].T @ q[b, rows, h, :])
    return dq_rows, dk_rows, dv_rows
