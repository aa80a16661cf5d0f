"""fp64 CPU oracle for the attention backward pass (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
module. It shares no code with the HIP path and never imports it.

The pages treat the backward pass as the training half of the same exact
attention: the intermediate matrices are not stored but recomputed on chip
when the gradients are formed ([JG] "Online softmax and recomputation"), and it
has been the harder part to make fast ([SN] "§2 Three core breakthroughs"; [LK]
"Key points" notes FA4 shipped without it). What it computes is the derivative
of the forward definition (oracle/exact.py) by the chain rule, written out in
float64 for one head, with dO the gradient arriving at O:

    P_ij  = exp(s_ij - LSE_i)              (0 for masked keys), s = scale * Q K^T
    dV    = P^T dO
    dP    = dO V^T
    D_i   = sum_j P_ij dP_ij  (= dO_i . O_i)
    dS_ij = P_ij (dP_ij - D_i)             (softmax Jacobian applied to dP)
    dQ    = scale * dS K
    dK    = scale * dS^T Q

Grouped-query heads (query head h reads key/value head h // (H / Hkv)): the
gradients of a shared key/value head are the sums over its query heads.
"""
from __future__ import annotations

import numpy as np

from .exact import _f64, kv_head


def _head_backward(qh, kh, vh, doh, causal, scale):
    """Gradients of one head: returns (dQ[N,d], dK[N,d], dV[N,d], D[N])."""
    n = qh.shape[0]
    s = scale * (qh @ kh.T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)          # softmax rows (exactly 0 where masked)
    dv = p.T @ doh
    dp = doh @ vh.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv, dd


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """Exact attention backward, float64.

    q, do: [B,H,N,d]; k, v: [B,Hkv,N,d] (Hkv divides H). Returns
    (dQ [B,H,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d], D [B,H,N]) with D_i = dO_i . O_i.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if do.shape != q.shape or k.shape != (B, Hkv, N, d) or v.shape != k.shape or Hkv < 1 or H % Hkv:
        raise ValueError(f"shapes q {q.shape} k {k.shape} v {v.shape} do {do.shape}")
    scale = float(np.float64(scale))
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            dq[b, h], dkh, dvh, dd[b, h] = _head_backward(q[b, h], k[b, g], v[b, g], do[b, h], causal, scale)
            dk[b, g] += dkh
            dv[b, g] += dvh
    return dq, dk, dv, dd


def attention_backward_rows(q, k, v, do, causal: bool, scale: float, picks_q, picks_kv):
    """Gradients at sampled rows only, for large shapes.

    picks_q: [(b, h, query rows)] -> dQ rows; picks_kv: [(b, g, key rows)] -> dK and
    dV rows of key/value head g (summed over its query heads). Every needed
    probability row or column is recomputed from the definition. Returns
    (list of dQ[len,d], list of (dK[len,d], dV[len,d])).
    """
    scale = float(np.float64(scale))
    H, Hkv = q.shape[1], k.shape[1]
    G = H // Hkv
    N = q.shape[2]
    out_q = []
    for b, h, rows in picks_q:
        rows = np.asarray(rows, dtype=np.int64)
        g = kv_head(h, H, Hkv)
        qh, kh, vh, doh = (_f64(t[b, x]) for t, x in ((q, h), (k, g), (v, g), (do, h)))
        p = _prob_rows(qh[rows], kh, rows, causal, scale)
        dp = doh[rows] @ vh.T
        dd = (p * dp).sum(axis=1)
        out_q.append(scale * ((p * (dp - dd[:, None])) @ kh))
    out_kv = []
    for b, g, rows in picks_kv:
        rows = np.asarray(rows, dtype=np.int64)
        kh, vh = _f64(k[b, g]), _f64(v[b, g])
        dk = np.zeros((rows.size, kh.shape[1]))
        dv = np.zeros((rows.size, kh.shape[1]))
        for h in range(g * G, g * G + G):
            qh, doh = _f64(q[b, h]), _f64(do[b, h])
            lse, dd = _row_stats(qh, kh, vh, doh, causal, scale)     # every query row
            s = scale * (qh @ kh[rows].T)                               # the picked key columns
            if causal:
                s = np.where(rows[None, :] <= np.arange(N)[:, None], s, -np.inf)
            ps = np.exp(s - lse[:, None])
            dps = doh @ vh[rows].T
            dv += ps.T @ doh
            dk += scale * ((ps * (dps - dd[:, None])).T @ qh)
        out_kv.append((dk, dv))
    return out_q, out_kv


def _row_stats(qh, kh, vh, doh, causal, scale, block=1024):
    """LSE_i and D_i = sum_j P_ij dP_ij of every query row, in row blocks (bounded memory)."""
    n = qh.shape[0]
    lse = np.empty(n)
    dd = np.empty(n)
    for r0 in range(0, n, block):
        rows = np.arange(r0, min(n, r0 + block))
        s = scale * (qh[rows] @ kh.T)
        if causal:
            s = np.where(np.arange(n)[None, :] <= rows[:, None], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        lse[rows] = m[:, 0] + np.log(z[:, 0])
        dd[rows] = ((e / z) * (doh[rows] @ vh.T)).sum(axis=1)
    return lse, dd


def _prob_rows(qrows, kh, rows, causal, scale):
    s = scale * (qrows @ kh.T)
    if causal:
        s = np.where(np.arange(kh.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_backward_varlen(q, k, v, do, cu_seqlens, causal: bool, scale: float):
    """Backward of packed variable-length attention (layout of oracle/exact.py's
    attention_varlen: q, do [H,total,d]; k, v [Hkv,total,d]; cu_seqlens [B+1]).

    Every sequence is the per-head backward above on its own rows and keys; key/value
    gradients of a shared head are summed over its query heads. Returns
    (dQ [H,total,d], dK [Hkv,total,d], dV [Hkv,total,d], D [H,total]).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    H, T, d = q.shape
    Hkv = k.shape[0]
    if do.shape != q.shape or k.shape != (Hkv, T, d) or v.shape != k.shape or Hkv < 1 or H % Hkv:
        raise ValueError(f"shapes q {q.shape} k {k.shape} v {v.shape} do {do.shape}")
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, not decrease and end at total")
    scale = float(np.float64(scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.zeros((H, T))
    for b in range(cu.size - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        if e == a:
            continue
        for h in range(H):
            g = kv_head(h, H, Hkv)
            dq[h, a:e], dkh, dvh, dd[h, a:e] = _head_backward(q[h, a:e], k[g, a:e], v[g, a:e], do[h, a:e], causal,
                                                               scale)
            dk[g, a:e] += dkh
            dv[g, a:e] += dvh
    return dq, dk, dv, dd
