"""fp64 CPU oracle for variable-length batches — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP library and its binding never do.

Source: the wmrh.cn FlashAttention v2 article, section 6 (future directions),
names variable-length sequences (with padding-aware scheduling) as the open
inefficiency of the method. The page defines no interface for it, so this
module fixes the plainest reading (also listed in the design notes):

  * a batch of B sequences is packed along the token axis: q, k, v, out, dout
    and the gradients are [T, H, d] with T = the total number of tokens, and
    ``cu_seqlens`` ([B + 1] integers, cu_seqlens[0] = 0, non-decreasing,
    cu_seqlens[B] = T) says that sequence b holds tokens
    cu_seqlens[b] .. cu_seqlens[b + 1] - 1; a sequence may be empty;
  * every sequence is its own attention problem: its queries see only its own
    keys, and query/key positions for the causal mask, the window and the ALiBi
    distance count from the sequence's first token;
  * queries and keys share the same sequence boundaries (self-attention);
  * the per-row logsumexp is stored [H, T] (head-major over the packed tokens).

So the oracle is the fixed-length definition (``oracle.attention``) applied to
each sequence's slice. No arithmetic of its own.
"""
from __future__ import annotations

import numpy as np

from . import attention as oa


def sequence_bounds(cu_seqlens):
    """[(start, end)] token ranges of the packed sequences (end exclusive)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]


def _one(x, a, e):
    """Tokens a..e-1 of a packed [T, H, d] array as a one-sequence batch [1, n, H, d]."""
    return x[None, a:e]


def varlen_forward(q, k, v, cu_seqlens, softmax_scale=None, causal=False, window_size=(-1, -1),
                   alibi_slopes=None):
    """Attention of every packed sequence on its own.

    q, k, v: [T, H, d]. Returns (out [T, H, d] float64, lse [H, T] float64).
    """
    q, k, v = oa.to_f64(q), oa.to_f64(k), oa.to_f64(v)
    T, H, _ = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(q.shape[-1])
    out = np.zeros((T, H, v.shape[-1]))
    lse = np.zeros((H, T))
    for a, e in sequence_bounds(cu_seqlens):
        if e <= a:
            continue
        o, l = oa.attention_forward(_one(q, a, e), _one(k, a, e), _one(v, a, e), softmax_scale, causal,
                                    window_size, alibi_slopes)
        out[a:e] = o[0]
        lse[:, a:e] = l[0]
    return out, lse


def varlen_backward(q, k, v, dout, cu_seqlens, softmax_scale=None, causal=False, window_size=(-1, -1),
                    alibi_slopes=None):
    """Gradients of sum(out * dout) for every packed sequence on its own. Returns (dq, dk, dv) [T, H, d]."""
    q, k, v, do = oa.to_f64(q), oa.to_f64(k), oa.to_f64(v), oa.to_f64(dout)
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(q.shape[-1])
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a, e in sequence_bounds(cu_seqlens):
        if e <= a:
            continue
        g = oa.attention_backward(_one(q, a, e), _one(k, a, e), _one(v, a, e), _one(do, a, e), softmax_scale,
                                  causal, window_size, alibi_slopes)
        dq[a:e], dk[a:e], dv[a:e] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


def _locate(cu_seqlens, t):
    """(sequence index, start, end) of packed token t."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    b = int(np.searchsorted(cu, t, side="right")) - 1
    while cu[b + 1] <= t:  # skip empty sequences that share the boundary
        b += 1
    return b, int(cu[b]), int(cu[b + 1])


def varlen_forward_rows(q, k, v, cu_seqlens, rows_ht, softmax_scale=None, causal=False,
                        window_size=(-1, -1), alibi_slopes=None):
    """The forward at sampled (head, packed token) rows. Returns (out [n, d], lse [n])."""
    q, k, v = oa.to_f64(q), oa.to_f64(k), oa.to_f64(v)
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(q.shape[-1])
    rows_ht = np.asarray(rows_ht)
    out = np.zeros((len(rows_ht), v.shape[-1]))
    lse = np.zeros(len(rows_ht))
    for n, (h, t) in enumerate(rows_ht):
        _, a, e = _locate(cu_seqlens, int(t))
        o, l = oa.attention_forward_rows(_one(q, a, e), _one(k, a, e), _one(v, a, e),
                                         np.array([[0, h, t - a]]), softmax_scale, causal, window_size,
                                         alibi_slopes)
        out[n], lse[n] = o[0], l[0]
    return out, lse


def varlen_backward_sampled(q, k, v, dout, cu_seqlens, q_rows_ht, k_rows_ht, softmax_scale=None,
                            causal=False, window_size=(-1, -1), alibi_slopes=None):
    """The backward at sampled (head, packed token) query rows (dQ) and key rows (dK, dV).

    Returns (dq_rows [n, d], dk_rows [m, d], dv_rows [m, d]).
    """
    q, k, v, do = oa.to_f64(q), oa.to_f64(k), oa.to_f64(v), oa.to_f64(dout)
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(q.shape[-1])
    q_rows_ht, k_rows_ht = np.asarray(q_rows_ht), np.asarray(k_rows_ht)
    d = q.shape[-1]
    dq_rows = np.zeros((len(q_rows_ht), d))
    dk_rows = np.zeros((len(k_rows_ht), d))
    dv_rows = np.zeros((len(k_rows_ht), v.shape[-1]))
    # group the requested rows by sequence so each sequence's full rows are formed once
    groups = {}
    for n, (h, t) in enumerate(q_rows_ht):
        groups.setdefault(_locate(cu_seqlens, int(t))[1:], ([], []))[0].append(n)
    for n, (h, t) in enumerate(k_rows_ht):
        groups.setdefault(_locate(cu_seqlens, int(t))[1:], ([], []))[1].append(n)
    for (a, e), (qs, ks) in groups.items():
        qsel = np.array([[0, q_rows_ht[n][0], q_rows_ht[n][1] - a] for n in qs], dtype=np.int64).reshape(-1, 3)
        ksel = np.array([[0, k_rows_ht[n][0], k_rows_ht[n][1] - a] for n in ks], dtype=np.int64).reshape(-1, 3)
        g = oa.attention_backward_sampled(_one(q, a, e), _one(k, a, e), _one(v, a, e), _one(do, a, e), qsel, ksel,
                                          softmax_scale, causal, window_size, alibi_slopes)
        dq_rows[qs], dk_rows[ks], dv_rows[ks] = g[0], g[1], g[2]
    return dq_rows, dk_rows, dv_rows
