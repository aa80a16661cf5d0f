"""Seeded synthetic workloads for the attention forward pass.

This module only draws inputs: it holds none of the attention arithmetic and
is the one piece shared by the tests, the benchmark, the oracle checks and the
GPU path. Every tensor is drawn on the CPU with torch's seeded generator in
float32 and rounded once to bfloat16 (round-to-nearest-even), so both sides see
bit-identical inputs.

Workloads (B heads-batch, H heads, N tokens, d head dim), all i.i.d. N(0,1):
  tiny      1 x  2 x   256 x  64  non-causal
  causal2k  4 x 16 x  2048 x 128  causal
  headline  2 x 32 x  8192 x 128  non-causal (the compute-bound shape)
  long32k   1 x 32 x 32768 x 128  causal
  drift8k   2 x 16 x  8192 x  64  causal, with a per-key logit drift: key j
            gets 0.002*j*u and every query gets u, u = ones(d)/sqrt(d), so the
            running row maximum keeps rising along the keys.
  gqa8k     2 x 32 x  8192 x 128  causal, grouped-query: 8 key/value heads,
            each shared by 4 consecutive query heads (k, v are [2, 8, 8192, 128]).

Variable-length batches (`draw_varlen`): sequences packed along the token axis
of a [H, total, d] tensor (k, v: [Hkv, total, d]) with cumulative lengths
cu_seqlens. `varlen_lengths` draws B lengths log-uniformly between lo and hi
(integers, so most are not multiples of any tile size).
  varlen    24 sequences of 64 .. 8192 tokens (seed 1007), 32 query heads,
            8 key/value heads, d = 128, causal.

FP8 inputs (`draw_fp8`): the same N(0,1) draws in float32, each tensor
quantised once to OCP e4m3 ("e4m3fn") codes with one per-tensor scale,
amax / 448 (448 is e4m3's largest finite value), by torch's round-to-nearest
conversion. V is handed over transposed, [B, H, d, ldv] with ldv = N rounded up
to a multiple of 16; columns N .. ldv-1 are padding that neither side reads.
  fp8_headline  2 x 32 x 8192 x 128 non-causal (seed 1003, the headline draw)
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    drift: bool
    seed: int
    Hkv: int = 0  # key/value heads; 0 means H (ordinary multi-head attention)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        """The float32 softmax scale 1/sqrt(d) handed to both sides."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def flops(self) -> float:
        """Attention flop count 4*B*H*N^2*d, halved for causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f


WORKLOADS = [
    Workload("tiny", 1, 2, 256, 64, False, False, 1001),
    Workload("causal2k", 4, 16, 2048, 128, True, False, 1002),
    Workload("headline", 2, 32, 8192, 128, False, False, 1003),
    Workload("long32k", 1, 32, 32768, 128, True, False, 1004),
    Workload("drift8k", 2, 16, 8192, 64, True, True, 1005),
    Workload("gqa8k", 2, 32, 8192, 128, True, False, 1006, Hkv=8),
]
BY_NAME = {w.name: w for w in WORKLOADS}

# Fewer query tiles (2 heads x 64 tiles of 256 rows) than the 256 compute units:
# the shape split keys are for.
LOWOCC = Workload("lowocc", 1, 2, 16384, 128, False, False, 1102)


def draw(B: int, H: int, N: int, d: int, seed: int, drift: bool = False,
         drift_rate: float = 0.002):
    """Draw (q, k, v) as bfloat16 CPU tensors [B,H,N,d], in that order, from one seed."""
    return draw_gqa(B, H, H, N, d, seed, drift, drift_rate)


def draw_gqa(B: int, H: int, Hkv: int, N: int, d: int, seed: int, drift: bool = False,
             drift_rate: float = 0.002):
    """Draw q [B,H,N,d] and k, v [B,Hkv,N,d] as bfloat16 CPU tensors, in that order.

    With Hkv = H this is exactly `draw`.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    if drift:
        u = torch.full((d,), 1.0 / math.sqrt(d), dtype=torch.float32)
        j = torch.arange(N, dtype=torch.float32).view(1, 1, N, 1)
        k += drift_rate * j * u
        q += u
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def varlen_lengths(B: int, lo: int, hi: int, seed: int) -> list[int]:
    """B sequence lengths, log-uniform on [lo, hi], from one seed."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    u = torch.rand((B,), generator=g, dtype=torch.float64)
    return [int(round(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u.tolist()]


def cu_seqlens(lengths) -> torch.Tensor:
    """Cumulative lengths [0, l0, l0+l1, ...] as an int32 CPU tensor."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def draw_varlen(lengths, H: int, Hkv: int, d: int, seed: int):
    """Packed sequences: q [H,total,d], k, v [Hkv,total,d] bf16 CPU tensors (drawn in
    that order, N(0,1) in fp32, rounded once) and cu_seqlens (int32 [B+1])."""
    cu = cu_seqlens(lengths)
    T = int(cu[-1])
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((H, T, d), generator=g, dtype=torch.float32)
    k = torch.randn((Hkv, T, d), generator=g, dtype=torch.float32)
    v = torch.randn((Hkv, T, d), generator=g, dtype=torch.float32)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), cu


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    name: str
    B: int
    lo: int
    hi: int
    H: int
    Hkv: int
    d: int
    causal: bool
    seed: int

    @property
    def lengths(self) -> list[int]:
        return varlen_lengths(self.B, self.lo, self.hi, self.seed)

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def flops(self) -> float:
        """Sum over sequences of 4*H*n^2*d, halved for causal."""
        f = sum(4.0 * self.H * n * n * self.d for n in self.lengths)
        return f / 2.0 if self.causal else f

    def inputs(self, seed: int | None = None):
        return draw_varlen(self.lengths, self.H, self.Hkv, self.d, self.seed if seed is None else seed)


VARLEN = VarlenWorkload("varlen", 24, 64, 8192, 32, 8, 128, True, 1007)


def workload_inputs(w: Workload, seed: int | None = None):
    """Inputs of a named workload (its own seed unless one is given)."""
    return draw_gqa(w.B, w.H, w.kv_heads, w.N, w.d, w.seed if seed is None else seed, w.drift)


E4M3_MAX = 448.0


def fp8_ldv(N: int) -> int:
    """Row length of the transposed V operand: N rounded up to a multiple of 16."""
    return (N + 15) // 16 * 16


def quantize_e4m3(x: torch.Tensor):
    """(codes, scale): x (float32) ~= decode(codes) * scale, with one float32 scale
    amax / 448 per tensor. Codes are uint8 e4m3fn bit patterns."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    scale = float(torch.tensor(amax / E4M3_MAX if amax > 0 else 1.0, dtype=torch.float32))
    y = (x / scale).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), scale


def draw_fp8(B: int, H: int, N: int, d: int, seed: int, drift: bool = False, pad_code: int = 0):
    """FP8 attention inputs from the same float32 draws as `draw` (same seed, same order):
    q8, k8 uint8 [B,H,N,d], vt8 uint8 [B,H,d,ldv] (V transposed, padding columns set to
    pad_code) and the three per-tensor scales (q_scale, k_scale, v_scale)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    if drift:
        u = torch.full((d,), 1.0 / math.sqrt(d), dtype=torch.float32)
        j = torch.arange(N, dtype=torch.float32).view(1, 1, N, 1)
        k += 0.002 * j * u
        q += u
    q8, qs = quantize_e4m3(q)
    k8, ks = quantize_e4m3(k)
    v8, vs = quantize_e4m3(v)
    ldv = fp8_ldv(N)
    vt8 = torch.full((B, H, d, ldv), pad_code, dtype=torch.uint8)
    vt8[..., :N] = v8.transpose(-1, -2)
    return q8, k8, vt8, (qs, ks, vs)


FP8_HEADLINE = Workload("fp8_headline", 2, 32, 8192, 128, False, False, 1003)


def digest(*tensors) -> str:
    """SHA-256 over the raw bytes of the given tensors (reproducibility record)."""
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
