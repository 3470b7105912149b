"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module. The product path (the HIP library and its Python binding) never
imports, calls or links it, and shares no code with it.

What it computes, and where that is stated
------------------------------------------
* "AI基础 | Flash Attention" (yeyulingfeng.com), sections "标准注意力矩阵计算很慢？"
  (why standard attention is slow) and "Tiling分块" (tiling): standard attention
  forms the N x N score matrix Q K^T, takes a row softmax of it and multiplies the
  result by V. Softmax is taken in two steps: find the row maximum, then divide
  exp(x - max) by the sum of those exponentials.
* The same page, section "Flash Attention背后的原理", and the FlashAttention-2 paper
  abstract ("FlashAttention-2: Faster Attention with Better Parallelism and Work
  Partitioning"): the tiled method computes exactly this result, with no
  approximation. So the oracle for the fast path is the plain definition.
* The wmrh.cn FlashAttention v2 article, section "5.1 API变更与兼容性" (API changes):
  the operation takes ``softmax_scale`` (None -> 1/sqrt(d)), ``causal``,
  ``window_size=(-1, -1)`` (local attention; -1 = unbounded) and
  ``alibi_slopes`` (linear position bias).
* "AI基础 | Flash Attention", section "反向传播" (backward): the forward keeps only
  per-row softmax statistics and the backward rebuilds the scores from them and
  Q, K, V. Here the saved statistic is the natural-log logsumexp per row, which
  fixes P = exp(S - LSE). The gradient formulas below are the chain rule applied
  to the definition; the pages do not print them.
* "AI基础 | Flash Attention", section "在线softmax" (online softmax): a running
  max, a running sum of exp(score - running max) and a running output of
  weighted V; when a block raises the max, the running sum and running output
  are rescaled. ``online_softmax_attention`` follows those steps, in the FA1 form
  (output kept normalised at every block) and in the FA2 form (section
  "Flash Attention2": the rescaling of the output is reduced and the division
  by the sum happens once at the end).

Readings of the pages (each is also listed in the design notes):
  * visibility of key j to query i: (not causal or j <= i) and
    (window_left < 0 or j >= i - window_left) and
    (window_right' < 0 or j <= i + window_right'), with window_right' = 0 when
    causal; bounds are inclusive and -1 means unbounded;
  * ALiBi enters after scaling and is not scaled: logit = scale*q.k - slope_h*|i-j|;
  * a row with no visible key (impossible for valid windows, because j = i is
    always visible) gets O = 0 and LSE = -inf;
  * layouts: q, k, v, out, dout and the gradients are [B, N, H, d]; lse is [B, H, N].

All arithmetic is float64. Inputs (numpy arrays or CPU torch tensors of any
float dtype, bf16 included) are upcast exactly.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024  # rows of the score matrix formed at a time (memory bound only)


def to_f64(x):
    """Exact upcast of a numpy array or CPU torch tensor (bf16/fp16/fp32/fp64) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.dtype != __import__("torch").float64:
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def visible(i, j, causal, window_left, window_right):
    """Boolean visibility of key position j to query position i (broadcasting)."""
    i = np.asarray(i)
    j = np.asarray(j)
    ok = np.ones(np.broadcast(i, j).shape, dtype=bool)
    right = 0 if causal else window_right
    if causal:
        ok &= j <= i
    if window_left >= 0:
        ok &= j >= i - window_left
    if right >= 0:
        ok &= j <= i + right
    return ok


def logits(q_rows, k_head, rows, scale, causal, window_left, window_right, slope):
    """Scaled, biased and masked scores of query rows `rows` against every key.

    q_rows: [n, d] float64, k_head: [N, d] float64, rows: [n] query positions.
    Returns [n, N] float64 with -inf where the key is not visible.
    """
    rows = np.asarray(rows)
    j = np.arange(k_head.shape[0])
    s = scale * (q_rows @ k_head.T)
    if slope is not None:
        s = s - slope * np.abs(rows[:, None] - j[None, :]).astype(np.float64)
    vis = visible(rows[:, None], j[None, :], causal, window_left, window_right)
    return np.where(vis, s, -np.inf)


def softmax_rows(s):
    """Row softmax of logits as the pages state it: row max first, then
    exp(x - max) divided by the sum of those exponentials.

    Returns (P, LSE) with LSE = max + ln(sum). Rows that are entirely -inf
    give P = 0 and LSE = -inf.
    """
    m = np.max(s, axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)  # exp(-inf) = 0 for invisible keys
    l = np.sum(e, axis=1, keepdims=True)
    l_safe = np.where(l > 0, l, 1.0)
    p = e / l_safe
    lse = (m_safe + np.log(l_safe))[:, 0]
    lse[empty] = -np.inf
    p[empty] = 0.0
    return p, lse


def _slope(alibi_slopes, h):
    return None if alibi_slopes is None else float(alibi_slopes[h])


def _prep(q, k, v, softmax_scale, window_size, alibi_slopes):
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(q.shape[-1])
    wl, wr = window_size
    slopes = to_f64(alibi_slopes)
    return q, k, v, float(softmax_scale), int(wl), int(wr), slopes


def attention_forward(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1),
                      alibi_slopes=None):
    """O = softmax(scale*Q K^T + bias, masked) V and the per-row LSE, by the definition.

    q, k, v: [B, N, H, d]. Returns (out [B, N, H, d] float64, lse [B, H, N] float64).
    """
    q, k, v, scale, wl, wr, slopes = _prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    B, N, H, d = q.shape
    out = np.zeros((B, N, H, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, :, h, :], v[b, :, h, :]
            for r0 in range(0, N, ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + ROW_CHUNK))
                s = logits(q[b, rows, h, :], kh, rows, scale, causal, wl, wr, _slope(slopes, h))
                p, lse_rows = softmax_rows(s)
                out[b, rows, h, :] = p @ vh
                lse[b, h, rows] = lse_rows
    return out, lse


def attention_forward_rows(q, k, v, rows_bhi, softmax_scale=None, causal=False,
                           window_size=(-1, -1), alibi_slopes=None):
    """The forward definition evaluated only at sampled query rows.

    rows_bhi: [n, 3] integer (b, h, i). Returns (out [n, d], lse [n]).
    """
    q, k, v, scale, wl, wr, slopes = _prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    rows_bhi = np.asarray(rows_bhi)
    out = np.zeros((len(rows_bhi), v.shape[-1]))
    lse = np.zeros(len(rows_bhi))
    for n, (b, h, i) in enumerate(rows_bhi):
        s = logits(q[b, i, h, :][None, :], k[b, :, h, :], np.array([i]), scale, causal, wl, wr,
                   _slope(slopes, h))
        p, l = softmax_rows(s)
        out[n] = (p @ v[b, :, h, :])[0]
        lse[n] = l[0]
    return out, lse


def _row_grads(s, p, do_rows, vh):
    """dP = dO V^T, D = rowsum(P * dP), dS = P * (dP - D) for a block of complete rows."""
    dp = do_rows @ vh.T
    dvec = np.sum(p * dp, axis=1, keepdims=True)
    return p * (dp - dvec), dvec[:, 0]


def attention_backward(q, k, v, dout, softmax_scale=None, causal=False, window_size=(-1, -1),
                       alibi_slopes=None):
    """Gradients of sum(O * dout) with respect to q, k, v, by the chain rule on the definition.

    dV = P^T dO;  dP = dO V^T;  D = rowsum(P * dP);  dS = P * (dP - D);
    dQ = scale * dS K;  dK = scale * dS^T Q.  (No gradient flows to the ALiBi slopes.)
    Returns (dq, dk, dv), each [B, N, H, d] float64.
    """
    q, k, v, scale, wl, wr, slopes = _prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    do = to_f64(dout)
    B, N, H, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
            for r0 in range(0, N, ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + ROW_CHUNK))
                s = logits(qh[rows], kh, rows, scale, causal, wl, wr, _slope(slopes, h))
                p, _ = softmax_rows(s)
                ds, _ = _row_grads(s, p, doh[rows], vh)
                dv[b, :, h, :] += p.T @ doh[rows]
                dq[b, rows, h, :] = scale * (ds @ kh)
                dk[b, :, h, :] += scale * (ds.T @ qh[rows])
    return dq, dk, dv


def attention_backward_sampled(q, k, v, dout, q_rows_bhi, k_rows_bhj, softmax_scale=None,
                               causal=False, window_size=(-1, -1), alibi_slopes=None):
    """The backward definition evaluated at sampled rows.

    dQ at query rows (b, h, i) needs only row i of P and dP. dK and dV at key rows
    (b, h, j) need column j of P and dS, hence every complete row of that head.
    Returns (dq_rows [n, d], dk_rows [m, d], dv_rows [m, d]).
    """
    q, k, v, scale, wl, wr, slopes = _prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    do = to_f64(dout)
    N = q.shape[1]
    q_rows_bhi = np.asarray(q_rows_bhi)
    k_rows_bhj = np.asarray(k_rows_bhj)
    dq_rows = np.zeros((len(q_rows_bhi), q.shape[-1]))
    for n, (b, h, i) in enumerate(q_rows_bhi):
        kh, vh = k[b, :, h, :], v[b, :, h, :]
        s = logits(q[b, i, h, :][None, :], kh, np.array([i]), scale, causal, wl, wr,
                   _slope(slopes, h))
        p, _ = softmax_rows(s)
        ds, _ = _row_grads(s, p, do[b, i, h, :][None, :], vh)
        dq_rows[n] = scale * (ds @ kh)[0]
    dk_rows = np.zeros((len(k_rows_bhj), k.shape[-1]))
    dv_rows = np.zeros((len(k_rows_bhj), v.shape[-1]))
    heads = sorted({(int(b), int(h)) for b, h, _ in k_rows_bhj})
    for (b, h) in heads:
        sel = np.nonzero((k_rows_bhj[:, 0] == b) & (k_rows_bhj[:, 1] == h))[0]
        js = k_rows_bhj[sel, 2]
        qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
        for r0 in range(0, N, ROW_CHUNK):
            rows = np.arange(r0, min(N, r0 + ROW_CHUNK))
            s = logits(qh[rows], kh, rows, scale, causal, wl, wr, _slope(slopes, h))
            p, _ = softmax_rows(s)
            ds, _ = _row_grads(s, p, doh[rows], vh)
            dv_rows[sel] += p[:, js].T @ doh[rows]
            dk_rows[sel] += scale * (ds[:, js].T @ qh[rows])
    return dq_rows, dk_rows, dv_rows


def online_softmax_attention(q, k, v, block, softmax_scale=None, causal=False,
                             window_size=(-1, -1), alibi_slopes=None, deferred=True):
    """Attention by the online-softmax recurrence over key blocks of size `block`.

    Steps, per query row and in the pages' terms:
      running_max m = -inf, running_sum l = 0, running_output acc = 0;
      for each key block: m_new = max(m, block max);
        l   = l * exp(m - m_new) + sum(exp(scores - m_new));
        acc = acc * exp(m - m_new) + sum(exp(scores - m_new) * v);
        (FA1 form, deferred=False: acc is kept divided by l after every block)
        m = m_new;
      a block seen while every score so far is -inf is skipped (nothing to add);
      output = acc / l (FA2 form), LSE = m + ln l.
    Meant for tiny inputs (Python loops over rows and blocks).
    Returns (out [B, N, H, d], lse [B, H, N]) in float64.
    """
    q, k, v, scale, wl, wr, slopes = _prep(q, k, v, softmax_scale, window_size, alibi_slopes)
    B, N, H, d = q.shape
    dv_ = v.shape[-1]
    out = np.zeros((B, N, H, dv_))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, :, h, :], v[b, :, h, :]
            for i in range(N):
                s_row = logits(q[b, i, h, :][None, :], kh, np.array([i]), scale, causal, wl, wr,
                               _slope(slopes, h))[0]
                m, l, acc = -np.inf, 0.0, np.zeros(dv_)
                for j0 in range(0, N, block):
                    sb = s_row[j0:j0 + block]
                    m_new = max(m, float(np.max(sb)))
                    if m_new == -np.inf:
                        continue
                    alpha = np.exp(m - m_new)  # exp(-inf) = 0 on the first visible block
                    e = np.exp(sb - m_new)
                    l_new = l * alpha + float(np.sum(e))
                    if deferred:
                        acc = acc * alpha + e @ vh[j0:j0 + block]
                    else:
                        acc = (acc * (l * alpha) + e @ vh[j0:j0 + block]) / l_new
                    m, l = m_new, l_new
                if l == 0.0:
                    out[b, i, h, :] = 0.0
                    lse[b, h, i] = -np.inf
                else:
                    out[b, i, h, :] = acc / l if deferred else acc
                    lse[b, h, i] = m + np.log(l)
    return out, lse
