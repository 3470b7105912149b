"""fp64 CPU oracle for block-sparse attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP library and its binding never do.

Source: the wmrh.cn FlashAttention v2 article, section 6 (future directions),
suggests combining the method with block-sparse patterns. The page fixes no
format, so this module states the plainest reading (also in the design notes):

  * a block mask of 0/1 bytes, one per (query block, key block) pair of
    BLOCK x BLOCK positions (BLOCK = 128), for every (batch, head):
    mask[b, h, i // BLOCK, j // BLOCK]; ``nb = ceil(N / BLOCK)`` blocks per side;
  * key j is visible to query i when the dense rule (causal, window) allows it
    AND the mask byte of its block pair is non-zero; ALiBi is unchanged;
  * a query row left with no visible key gets O = 0 and LSE = -inf, and its
    gradients are zero (the defensive convention of the dense oracle, which a
    sparse mask can reach).

The arithmetic is the dense definition (``oracle.attention``): the same scores,
with the extra -inf entries, through the same row softmax and chain rule.
"""
from __future__ import annotations

import numpy as np

from . import attention as oa

BLOCK = 128


def key_mask_rows(block_mask_bh, rows, N, block=BLOCK):
    """Boolean [len(rows), N]: the block-mask term for query positions `rows`."""
    rows = np.asarray(rows)
    m = np.asarray(block_mask_bh) != 0
    return m[rows // block][:, np.arange(N) // block]


def _masked_logits(q_rows, kh, rows, scale, causal, wl, wr, slope, block_mask_bh):
    s = oa.logits(q_rows, kh, rows, scale, causal, wl, wr, slope)
    return np.where(key_mask_rows(block_mask_bh, rows, kh.shape[0]), s, -np.inf)


def _mask_of(block_mask, b, h):
    return np.asarray(block_mask)[b, h]


def blocksparse_forward(q, k, v, block_mask, softmax_scale=None, causal=False, window_size=(-1, -1),
                        alibi_slopes=None):
    """q, k, v: [B, N, H, d]; block_mask: [B, H, nb, nb]. Returns (out [B, N, H, d], lse [B, H, N])."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    B, N, H, _ = q.shape
    out = np.zeros((B, N, H, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, :, h, :], v[b, :, h, :]
            for r0 in range(0, N, oa.ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + oa.ROW_CHUNK))
                s = _masked_logits(q[b, rows, h, :], kh, rows, scale, causal, wl, wr, oa._slope(slopes, h),
                                   _mask_of(block_mask, b, h))
                p, lse_rows = oa.softmax_rows(s)
                out[b, rows, h, :] = p @ vh
                lse[b, h, rows] = lse_rows
    return out, lse


def blocksparse_backward(q, k, v, dout, block_mask, softmax_scale=None, causal=False, window_size=(-1, -1),
                         alibi_slopes=None):
    """Gradients of sum(out * dout) under the block mask. Returns (dq, dk, dv) [B, N, H, d]."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    do = oa.to_f64(dout)
    B, N, H, _ = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
            for r0 in range(0, N, oa.ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + oa.ROW_CHUNK))
                s = _masked_logits(qh[rows], kh, rows, scale, causal, wl, wr, oa._slope(slopes, h),
                                   _mask_of(block_mask, b, h))
                p, _ = oa.softmax_rows(s)
                ds, _ = oa._row_grads(s, p, doh[rows], vh)
                dv[b, :, h, :] += p.T @ doh[rows]
                dq[b, rows, h, :] = scale * (ds @ kh)
                dk[b, :, h, :] += scale * (ds.T @ qh[rows])
    return dq, dk, dv


def blocksparse_forward_rows(q, k, v, block_mask, rows_bhi, softmax_scale=None, causal=False,
                             window_size=(-1, -1), alibi_slopes=None):
    """The forward at sampled (b, h, i) rows. Returns (out [n, d], lse [n])."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    rows_bhi = np.asarray(rows_bhi)
    out = np.zeros((len(rows_bhi), v.shape[-1]))
    lse = np.zeros(len(rows_bhi))
    for n, (b, h, i) in enumerate(rows_bhi):
        s = _masked_logits(q[b, i, h, :][None, :], k[b, :, h, :], np.array([i]), scale, causal, wl, wr,
                           oa._slope(slopes, h), _mask_of(block_mask, b, h))
        p, l = oa.softmax_rows(s)
        out[n] = (p @ v[b, :, h, :])[0]
        lse[n] = l[0]
    return out, lse


def blocksparse_backward_sampled(q, k, v, dout, block_mask, q_rows_bhi, k_rows_bhj, softmax_scale=None,
                                 causal=False, window_size=(-1, -1), alibi_slopes=None):
    """The backward at sampled query rows (dQ) and key rows (dK, dV); key rows need
    every complete row of their head. Returns (dq_rows [n, d], dk_rows [m, d], dv_rows [m, d])."""
    q, k, v, scale, wl, wr, slopes = oa._prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    do = oa.to_f64(dout)
    N = q.shape[1]
    q_rows_bhi, k_rows_bhj = np.asarray(q_rows_bhi), np.asarray(k_rows_bhj)
    dq_rows = np.zeros((len(q_rows_bhi), q.shape[-1]))
    for n, (b, h, i) in enumerate(q_rows_bhi):
        kh, vh = k[b, :, h, :], v[b, :, h, :]
        s = _masked_logits(q[b, i, h, :][None, :], kh, np.array([i]), scale, causal, wl, wr, oa._slope(slopes, h),
                           _mask_of(block_mask, b, h))
        p, _ = oa.softmax_rows(s)
        ds, _ = oa._row_grads(s, p, do[b, i, h, :][None, :], vh)
        dq_rows[n] = scale * (ds @ kh)[0]
    dk_rows = np.zeros((len(k_rows_bhj), k.shape[-1]))
    dv_rows = np.zeros((len(k_rows_bhj), v.shape[-1]))
    for (b, h) in sorted({(int(b), int(h)) for b, h, _ in k_rows_bhj}):
        sel = np.nonzero((k_rows_bhj[:, 0] == b) & (k_rows_bhj[:, 1] == h))[0]
        js = k_rows_bhj[sel, 2]
        qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
        for r0 in range(0, N, oa.ROW_CHUNK):
            rows = np.arange(r0, min(N, r0 + oa.ROW_CHUNK))
            s = _masked_logits(qh[rows], kh, rows, scale, causal, wl, wr, oa._slope(slopes, h),
                               _mask_of(block_mask, b, h))
            p, _ = oa.softmax_rows(s)
            ds, _ = oa._row_grads(s, p, doh[rows], vh)
            dv_rows[sel] += p[:, js].T @ doh[rows]
            dk_rows[sel] += scale * (ds[:, js].T @ qh[rows])
    return dq_rows, dk_rows, dv_rows
