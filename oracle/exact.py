"""fp64 CPU oracle for the exact attention forward pass (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
module. It shares no code with the HIP path and never imports it.

Pages cited (titles as printed, sections as headed on each page):
  [LK] "FlashAttention 4: faster, more memory-efficient attention for LLMs"
       (ja.linux-konsole.com)
  [JG] "Flash Attention" glossary entry (jisaku.com)
  [SN] "FlashAttention-4: algorithm-kernel fused pipeline for asymmetric
       hardware scaling" (sns.style)

What is computed ([LK] "Introduction"): queries are multiplied with keys, the
result is normalised by a softmax and multiplied with the values. The method
is exact, not an approximation ([JG] "Summary of optimisations", last bullet),
so the oracle is that definition evaluated in float64:

    s_ij  = scale * sum_k q_ik k_jk                 for j in J(i)
    m_i   = max_j s_ij,  l_i = sum_j exp(s_ij - m_i)
    O_i   = sum_j exp(s_ij - m_i) / l_i * v_j
    LSE_i = m_i + ln(l_i)                           (natural log, scale included)

J(i) = all keys (non-causal) or keys j <= i (causal, lower-triangular mask).
Inputs are widened exactly to float64 (bfloat16 and float32 values are exact
in float64), and `scale` is the float32 value the kernel uses, widened.

Grouped-query attention (`attention_gqa`): several query heads share one key and
value head ([LK] "Key points" and "Compatibility and current status", which name
GQA/MQA among the configurations earlier FlashAttention versions supported).
The pages do not say which query heads share a key/value head; the reading used
here is consecutive groups: with H query heads and Hkv key/value heads (Hkv
divides H), query head h reads key/value head floor(h / (H / Hkv)). MQA is
Hkv = 1; Hkv = H is ordinary multi-head attention.

Variable-length batches (`attention_varlen`): several sequences of different
lengths packed along the token axis, the other feature [LK] "Key points" lists
as missing from FA4. The pages give no layout; the reading used here is the
dense layout with the batch folded into the token axis: q is [H, total, d],
k and v are [Hkv, total, d], and sequence b owns tokens cu[b] .. cu[b+1]-1 of
every head (cu = cumulative lengths, cu[0] = 0, cu[B] = total). A query attends
only to the keys of its own sequence; the causal mask compares positions inside
the sequence. Query and key sequences share the same bounds (self-attention).
LSE is [H, total].

`tiled_online_attention` is a second, test-only float64 model that follows the
algorithm the pages describe: tiles of queries and keys, a running maximum and
running sum per query row ([JG] "Online softmax and recomputation";
[LK] "Why attention kernels still dominate LLM cost"), and the adaptive policy
that rescales only when the new maximum exceeds the one in use by more than a
threshold ([LK] "Smarter online softmax rescaling (new in FA4)"). It works in
base 2 because the pages name exp2 ([LK] "Software exponential on CUDA cores").
It pins the algebra of lazy rescaling against `attention`; it is not used to
produce expected values for the GPU.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def _f64(x) -> np.ndarray:
    """Widen to float64 (exact for bf16/fp32); accepts numpy arrays or torch CPU tensors."""
    if hasattr(x, "detach"):  # torch tensor: go through float32, which holds bf16 exactly
        x = x.detach().to("cpu").float().numpy()
    a = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle inputs must be finite")
    return a


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"expected equal [B,H,N,d] shapes, got {q.shape} {k.shape} {v.shape}")


def _rows_of_head(qh, kh, vh, rows, causal, scale):
    """Definition for the query rows `rows` of one head: returns (O[len(rows),d], LSE[len(rows)])."""
    s = scale * (qh[rows] @ kh.T)                      # [R, N] scores, scale included
    if causal:
        keys = np.arange(kh.shape[0])[None, :]
        s = np.where(keys <= np.asarray(rows)[:, None], s, -np.inf)   # key j visible iff j <= i
    m = s.max(axis=1, keepdims=True)                   # row maximum (finite: key 0 always visible)
    e = np.exp(s - m)                                  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1, keepdims=True)
    o = (e @ vh) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention(q, k, v, causal: bool, scale: float, row_block: int = 1024):
    """Exact attention forward, float64. q, k, v: [B,H,N,d]. Returns (O[B,H,N,d], LSE[B,H,N]).

    Rows are evaluated in blocks of `row_block` only to bound memory; every row's
    arithmetic is the definition above, independent of the blocking.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_shapes(q, k, v)
    scale = float(np.float64(scale))
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                o[b, h, rows], lse[b, h, rows] = _rows_of_head(q[b, h], k[b, h], v[b, h], rows, causal, scale)
    return o, lse


def _check_gqa_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError(f"expected q [B,H,N,d] and k, v [B,Hkv,N,d], got {q.shape} {k.shape} {v.shape}")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or k.shape[1] < 1 or H % k.shape[1]:
        raise ValueError(f"key/value heads {k.shape[1]} must divide query heads {H}; shapes {q.shape} {k.shape}")


def kv_head(h: int, H: int, Hkv: int) -> int:
    """Key/value head read by query head h (consecutive groups of H / Hkv query heads)."""
    return h // (H // Hkv)


def attention_gqa(q, k, v, causal: bool, scale: float, row_block: int = 1024):
    """Exact grouped-query attention forward, float64. q: [B,H,N,d]; k, v: [B,Hkv,N,d].

    Each query head is the definition above evaluated against its key/value head.
    Returns (O[B,H,N,d], LSE[B,H,N]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_gqa_shapes(q, k, v)
    scale = float(np.float64(scale))
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                o[b, h, rows], lse[b, h, rows] = _rows_of_head(q[b, h], k[b, g], v[b, g], rows, causal, scale)
    return o, lse


def attention_gqa_rows(q, k, v, causal: bool, scale: float, picks):
    """`attention_gqa` evaluated only at sampled outputs (picks as in `attention_rows`)."""
    scale = float(np.float64(scale))
    H, Hkv = q.shape[1], k.shape[1]
    out = []
    for b, h, rows in picks:
        g = kv_head(h, H, Hkv)
        qh, kh, vh = _f64(q[b, h]), _f64(k[b, g]), _f64(v[b, g])
        out.append(_rows_of_head(qh, kh, vh, np.asarray(rows, dtype=np.int64), causal, scale))
    return out


def _check_varlen(q, k, v, cu):
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape:
        raise ValueError(f"expected q [H,total,d] and k, v [Hkv,total,d], got {q.shape} {k.shape} {v.shape}")
    H, T, d = q.shape
    if k.shape[1] != T or k.shape[2] != d or k.shape[0] < 1 or H % k.shape[0]:
        raise ValueError(f"key/value shape {k.shape} does not fit queries {q.shape}")
    cu = np.asarray(cu, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError(f"cu_seqlens must start at 0, not decrease and end at total={T}: {cu.tolist()[:8]}...")
    return cu


def attention_varlen(q, k, v, cu_seqlens, causal: bool, scale: float, row_block: int = 1024):
    """Exact attention over packed variable-length sequences, float64.

    q: [H,total,d]; k, v: [Hkv,total,d] (Hkv divides H; query head h reads key/value
    head h // (H // Hkv)); cu_seqlens: B+1 cumulative lengths. Each sequence is the
    definition above on its own rows and keys. Returns (O[H,total,d], LSE[H,total]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = _check_varlen(q, k, v, cu_seqlens)
    scale = float(np.float64(scale))
    H, T, d = q.shape
    Hkv = k.shape[0]
    o = np.empty((H, T, d))
    lse = np.empty((H, T))
    for b in range(cu.size - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, e - a, row_block):
                rows = np.arange(r0, min(e - a, r0 + row_block))
                o[h, a + rows], lse[h, a + rows] = _rows_of_head(q[h, a:e], k[g, a:e], v[g, a:e], rows, causal, scale)
    return o, lse


def attention_varlen_rows(q, k, v, cu_seqlens, causal: bool, scale: float, picks):
    """`attention_varlen` at sampled outputs: picks = [(h, token indices)], tokens
    in [0, total) (any sequences). Returns [(O[len,d], LSE[len])]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    scale = float(np.float64(scale))
    H, Hkv = q.shape[0], k.shape[0]
    out = []
    for h, toks in picks:
        toks = np.asarray(toks, dtype=np.int64)
        g = kv_head(h, H, Hkv)
        o = np.empty((toks.size, q.shape[2]))
        lse = np.empty(toks.size)
        seq = np.searchsorted(cu, toks, side="right") - 1   # sequence b with cu[b] <= t < cu[b+1]
        for b in np.unique(seq):
            a, e = int(cu[b]), int(cu[b + 1])
            sel = seq == b
            qh, kh, vh = _f64(q[h, a:e]), _f64(k[g, a:e]), _f64(v[g, a:e])
            o[sel], lse[sel] = _rows_of_head(qh, kh, vh, toks[sel] - a, causal, scale)
        out.append((o, lse))
    return out


def attention_rows(q, k, v, causal: bool, scale: float, picks):
    """Definition evaluated only at sampled outputs.

    picks: iterable of (b, h, rows) with rows a sequence of query indices.
    Returns a list of (O[len(rows),d], LSE[len(rows)]) in the same order.
    Used where the full shape would take the CPU too long; each sampled row is
    computed exactly as in `attention`.
    """
    scale = float(np.float64(scale))
    out = []
    for b, h, rows in picks:
        qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
        rows = np.asarray(rows, dtype=np.int64)
        out.append(_rows_of_head(qh, kh, vh, rows, causal, scale))
    return out


def attention_probs(q, k, causal: bool, scale: float):
    """The full softmax matrix P[B,H,N,N] (tiny shapes only), for invariant checks."""
    q, k = _f64(q), _f64(k)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        n = q.shape[2]
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def brute_force_attention(q, k, v, causal: bool, scale: float):
    """Pure-Python loops with math.exp over nested lists; tiny inputs only.

    Written without the max shift (plain exp(s)/sum exp(s)), so it also pins
    that the shifted form used above is the same function.
    """
    q, k, v = (_f64(t).tolist() for t in (q, k, v))
    scale = float(np.float64(scale))
    B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    o = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                w = []
                for j in keys:
                    s = 0.0
                    for c in range(d):
                        s += q[b][h][i][c] * k[b][h][j][c]
                    w.append(math.exp(scale * s))
                z = sum(w)
                for c in range(d):
                    o[b][h][i][c] = sum(wj * v[b][h][j][c] for wj, j in zip(w, keys)) / z
                lse[b][h][i] = math.log(z)
    return np.array(o), np.array(lse)


def brute_force_attention_gqa(q, k, v, causal: bool, scale: float):
    """Pure-Python loops for grouped-query attention (tiny inputs only), without the
    max shift. The head map is walked from the key/value side: key/value head g
    serves the query heads g*G .. g*G + G - 1, G = H / Hkv."""
    q, k, v = (_f64(t).tolist() for t in (q, k, v))
    scale = float(np.float64(scale))
    B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = H // Hkv
    o = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for g in range(Hkv):
            for h in range(g * G, g * G + G):
                for i in range(N):
                    keys = range(i + 1) if causal else range(N)
                    w = [math.exp(scale * sum(q[b][h][i][c] * k[b][g][j][c] for c in range(d))) for j in keys]
                    z = sum(w)
                    for c in range(d):
                        o[b][h][i][c] = sum(wj * v[b][g][j][c] for wj, j in zip(w, keys)) / z
                    lse[b][h][i] = math.log(z)
    return np.array(o), np.array(lse)


def brute_force_attention_varlen(q, k, v, cu_seqlens, causal: bool, scale: float):
    """Pure-Python loops over packed sequences (tiny inputs only), without the max
    shift. Every (query token, key token) pair of a head is visited; a key counts
    when both tokens lie in the same sequence (found by scanning the bounds) and,
    if causal, the key does not come after the query."""
    q, k, v = (_f64(t).tolist() for t in (q, k, v))
    bounds = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    scale = float(np.float64(scale))
    H, T, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)

    def seq_of(t):
        for b in range(len(bounds) - 1):
            if bounds[b] <= t < bounds[b + 1]:
                return b
        raise ValueError(t)

    o = [[[0.0] * d for _ in range(T)] for _ in range(H)]
    lse = [[0.0] * T for _ in range(H)]
    for h in range(H):
        g = h * Hkv // H
        for i in range(T):
            keys = [j for j in range(T) if seq_of(j) == seq_of(i) and (not causal or j <= i)]
            w = [math.exp(scale * sum(q[h][i][c] * k[g][j][c] for c in range(d))) for j in keys]
            z = sum(w)
            for c in range(d):
                o[h][i][c] = sum(wj * v[g][j][c] for wj, j in zip(w, keys)) / z
            lse[h][i] = math.log(z)
    return np.array(o), np.array(lse)


def tiled_online_attention(q, k, v, causal: bool, scale: float, br: int, bc: int, tau: float):
    """Test-only float64 model of tiled attention with an online, lazily rescaled softmax.

    Follows the pages' algorithm: each block of `br` query rows streams the keys
    and values in tiles of `bc`, keeping per row a running maximum and a running
    sum ([JG] "Online softmax and recomputation"); the exponentials are taken in
    base 2 ([LK] "Software exponential on CUDA cores"); the stored maximum and
    the partial results are only rescaled when the tile's maximum exceeds the
    maximum in use by more than `tau` (log2 units), the adaptive policy of
    [LK] "Smarter online softmax rescaling (new in FA4)". tau = 0 is the
    classic policy (rescale on every increase).

    Returns (O, LSE, rescale_events[B,H,N]); the events count the rescales
    after a row's first tile (which always initialises the row).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_shapes(q, k, v)
    scale = float(np.float64(scale))
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    events = np.zeros((B, H, N), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N, br):
                rows = np.arange(i0, min(N, i0 + br))
                qi = q[b, h, rows]
                m_used = np.full(len(rows), -np.inf)   # max in use, log2 units
                l = np.zeros(len(rows))                # running sum of 2^(x - m_used)
                acc = np.zeros((len(rows), d))         # running sum of 2^(x - m_used) v
                first = np.ones(len(rows), dtype=bool)
                for j0 in range(0, N, bc):
                    keys = np.arange(j0, min(N, j0 + bc))
                    if causal and keys[0] > rows[-1]:
                        break                          # tiles above the diagonal hold no visible key
                    x = (scale * (qi @ k[b, h, keys].T)) * LOG2E   # scaled logits, base 2
                    if causal:
                        x = np.where(keys[None, :] <= rows[:, None], x, -np.inf)
                    m_tile = x.max(axis=1)
                    grow = m_tile - m_used             # +inf on a row's first visible tile
                    redo = grow > tau
                    if np.any(redo):
                        m_new = np.where(redo, m_tile, m_used)
                        alpha = np.exp2(m_used - m_new)    # 0 on first tile, 1 where not redone
                        acc *= alpha[:, None]
                        l *= alpha
                        events[b, h, rows] += (redo & ~first).astype(np.int64)
                        first &= ~(redo & np.isfinite(m_new))
                        m_used = m_new
                    p = np.exp2(x - m_used[:, None])   # <= 2^tau where the maximum was not refreshed
                    l += p.sum(axis=1)
                    acc += p @ v[b, h, keys]
                o[b, h, rows] = acc / l[:, None]
                lse[b, h, rows] = LN2 * (m_used + np.log2(l))
    return o, lse, events
