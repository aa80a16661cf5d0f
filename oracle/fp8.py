"""fp64 CPU oracle for FP8 attention forward (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
module. It shares no code with the HIP path and never imports it.

The FP8 variant of the method (page "Flash Attention" glossary, section
"FlashAttention-3 and the FP8 era", and its hardware section on the H100's FP8
and the B200's low-precision formats) runs the two products on 8-bit
floating-point inputs.
The pages give neither the format nor the scaling; the readings used here:

  * inputs are OCP e4m3 ("e4m3fn") codes: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
    m/8 * 2^-6; the pattern S.1111.111 is NaN; there are no infinities, so the
    largest finite magnitude is 1.75 * 2^8 = 448;
  * each tensor carries one float32 dequantisation scale: the real value of a
    code c is decode(c) * scale;
  * V is handed over transposed, [B, H, d, ldv] (ldv >= N; columns past N are
    padding and are never read).

The method is still exact attention of those real values, so the oracle
decodes the codes, applies the scales and evaluates the float64 definition of
`exact.attention`.

`fp8_error_bound` states how far an FP8 kernel may lie from that exact value.
Three roundings separate them, each bounded from the arithmetic:
  (1) the matrix core's dot products of e4m3 values: every product of two
      e4m3 values is exact in fp32, but the accumulation inside one matrix
      instruction is not an fp32 sum; its error is taken as at most
      EPS_DOT * sum_k |q_k k_k| (relative to the sum of the absolute terms).
      A score error |ds| <= E moves each probability by a factor within
      e^(+-2E) and the LSE by at most E;
  (2) P rounded to e4m3 before the second product: relative error at most
      2^-4 for values at or above 2^-6 (three mantissa bits, round to nearest)
      and absolute error at most 2^-10 below (subnormal spacing 2^-9). The
      kernel's P is 2^(x - m_used) with m_used never above the row maximum,
      so in the oracle's units the absolute part is at most 2^-10 / l_i;
  (3) O rounded to bf16 on store: relative 2^-9.
The row sum is formed from the fp32 probabilities before their rounding, so
(2) does not enter the LSE.
"""
from __future__ import annotations

import numpy as np

from .exact import attention, attention_rows

E4M3_BIAS = 7
E4M3_MAX = 448.0
# Bound (1): score error of one e4m3 dot product relative to sum_k |q_k k_k|.
# The gfx950 matrix core was measured at <= 2^-11.60 over 4.2 million dot
# products of codes spread uniformly over the whole e4m3 range (the worst case
# for alignment inside the instruction); 2^-10 leaves a factor of 3.1.
EPS_DOT = 2.0 ** -10
P_REL = 2.0 ** -4      # e4m3 relative rounding bound for normal values
P_ABS = 2.0 ** -10     # e4m3 absolute rounding bound below 2^-6
O_REL = 2.0 ** -9      # bf16 relative rounding bound


def e4m3_decode(codes) -> np.ndarray:
    """Real values (float64) of e4m3fn bit patterns (any integer array of 0..255).

    Written from the field layout: sign s = bit 7, exponent e = bits 6..3,
    mantissa m = bits 2..0. e == 0: (-1)^s * m/8 * 2^(1-7); otherwise
    (-1)^s * (1 + m/8) * 2^(e-7); e == 15 and m == 7: NaN.
    """
    c = np.asarray(codes, dtype=np.int64)
    if c.size and (c.min() < 0 or c.max() > 255):
        raise ValueError("e4m3 codes are bytes")
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - E4M3_BIAS)
    sub = (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def _tensor_np(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x)


def dequantize(q8, k8, vt8, N: int, scales):
    """float64 q, k, v [B,H,N,d] from the codes and per-tensor scales (q_scale, k_scale, v_scale).
    vt8 is [B,H,d,ldv]; only its first N columns are read."""
    qs, ks, vs = (float(np.float32(s)) for s in scales)
    q = e4m3_decode(_tensor_np(q8)) * qs
    k = e4m3_decode(_tensor_np(k8)) * ks
    vt = _tensor_np(vt8)
    if vt.ndim != 4 or vt.shape[-1] < N:
        raise ValueError(f"vt must be [B,H,d,ldv] with ldv >= N, got {vt.shape}")
    v = np.swapaxes(e4m3_decode(vt[..., :N]), -1, -2) * vs
    for name, a in (("q", q), ("k", k), ("v", v)):
        if not np.all(np.isfinite(a)):
            raise ValueError(f"{name} holds NaN codes")
    return q, k, v


def attention_fp8(q8, k8, vt8, scales, causal: bool, scale: float):
    """Exact attention (float64) of the dequantised FP8 inputs: (O[B,H,N,d], LSE[B,H,N])."""
    N = _tensor_np(q8).shape[2]
    q, k, v = dequantize(q8, k8, vt8, N, scales)
    return attention(q, k, v, causal, scale)


def attention_fp8_rows(q8, k8, vt8, scales, causal: bool, scale: float, picks):
    """`attention_fp8` at sampled outputs (picks as in `exact.attention_rows`)."""
    N = _tensor_np(q8).shape[2]
    q, k, v = dequantize(q8, k8, vt8, N, scales)
    return attention_rows(q, k, v, causal, scale, picks)


def _bound_rows(qh, kh, vh, rows, causal, scale):
    """Per-row (O bound, LSE bound) of one head for the query rows `rows` (see module doc)."""
    s = scale * (qh[rows] @ kh.T)
    t = abs(scale) * (np.abs(qh[rows]) @ np.abs(kh.T))      # sum_k |scale q_k k_k|
    vis = np.ones_like(s, dtype=bool)
    if causal:
        vis = np.arange(kh.shape[0])[None, :] <= np.asarray(rows)[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1)
    p = e / l[:, None]
    E = EPS_DOT * np.where(vis, t, 0.0).max(axis=1)          # bound (1) on every score of the row
    av = np.abs(vh)
    o = p @ vh
    grow = np.exp(2.0 * E)
    term_dot = (grow - 1.0)[:, None] * (p @ av)              # (1): P within a factor e^(+-2E)
    term_p = (P_REL * grow)[:, None] * (p @ av) + (P_ABS / l)[:, None] * (np.where(vis, 1.0, 0.0) @ av)  # (2)
    bo = term_dot + term_p
    bo = bo + O_REL * (np.abs(o) + bo)                       # (3)
    return bo.max(axis=1), E


def fp8_error_bound(q8, k8, vt8, scales, causal: bool, scale: float):
    """Per-row bounds (bound_O[B,H,N] on max_k |O_ik - O_ref,ik|, bound_LSE[B,H,N]) for an FP8
    kernel against `attention_fp8` (module doc: roundings (1)-(3))."""
    N = _tensor_np(q8).shape[2]
    q, k, v = dequantize(q8, k8, vt8, N, scales)
    B, H = q.shape[:2]
    bo = np.empty((B, H, N))
    bl = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, 1024):
                rows = np.arange(r0, min(N, r0 + 1024))
                bo[b, h, rows], bl[b, h, rows] = _bound_rows(q[b, h], k[b, h], v[b, h], rows, causal, scale)
    return bo, bl


def fp8_error_bound_rows(q8, k8, vt8, scales, causal: bool, scale: float, picks):
    """`fp8_error_bound` at sampled rows: picks = [(b, h, row indices)]; returns lists of arrays."""
    N = _tensor_np(q8).shape[2]
    q, k, v = dequantize(q8, k8, vt8, N, scales)
    out = []
    for b, h, rows in picks:
        out.append(_bound_rows(q[b, h], k[b, h], v[b, h], np.asarray(rows), causal, scale))
    return out


def brute_force_attention_fp8(q8, k8, vt8, scales, causal: bool, scale: float, decode):
    """Pure-Python loops (tiny inputs only) reading the codes through `decode` (a callable
    code -> float supplied by the caller, e.g. torch's own e4m3fn conversion), with no max
    shift: O_i = sum_j w_ij v_j / sum_j w_ij, w_ij = exp(s_ij), LSE_i = ln sum_j w_ij."""
    import math
    q8, k8, vt8 = (_tensor_np(x).tolist() for x in (q8, k8, vt8))
    qs, ks, vs = (float(np.float32(s)) for s in scales)
    sc = float(np.float32(scale))
    B, H, N, d = len(q8), len(q8[0]), len(q8[0][0]), len(q8[0][0][0])
    O = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                tot = 0.0
                acc = [0.0] * d
                for j in range(N):
                    if causal and j > i:
                        continue
                    s = sc * sum(decode(q8[b][h][i][x]) * qs * decode(k8[b][h][j][x]) * ks for x in range(d))
                    w = math.exp(s)
                    tot += w
                    for x in range(d):
                        acc[x] += w * decode(vt8[b][h][x][j]) * vs
                O[b][h][i] = [a / tot for a in acc]
                L[b][h][i] = math.log(tot)
    return np.array(O), np.array(L)
