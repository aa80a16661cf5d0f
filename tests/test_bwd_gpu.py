"""HIP attention backward vs the fp64 oracle, through the C ABI (MI355X only).

The GPU forward pass supplies O and LSE (as in training); the oracle computes
dQ, dK, dV and D from q, k, v and dO alone. Tolerance, from the arithmetic: P
and dS are rounded to bf16 before their products (relative 2^-9 per term), the
outputs are rounded to bf16 (2^-9), O enters D in bf16 and LSE comes from the
forward pass in fp32. Rows of dS sum to zero, so dQ and dK are differences of
terms that can each be several times larger than the result; a few 2^-9
roundings on such terms give errors of a few 2^-9 of the tensor's size. Each
gradient tensor (and D) must satisfy max|X - X_ref| <= 2e-2 * max|X_ref|
(2e-2 is about ten roundings of 2^-9; measured errors stay below 1e-2).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import device, note

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2


def rel_err(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-30)) if ref.size else 0.0


def run_gpu_backward(q, k, v, do, causal, scale):
    dev = device()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = binding.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, delta = binding.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv, delta))


def draw(B, H, Hkv, N, d, seed):
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=seed)
    do = inputs.draw(B, H, N, d, seed=seed + 7919)[0]
    return q, k, v, do


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (1, 2, 2, 256, 64, False),
    (1, 2, 2, 256, 64, True),
    (2, 4, 2, 300, 128, True),
    (1, 4, 1, 129, 128, False),
    (1, 2, 2, 1, 64, True),
    (1, 3, 3, 33, 128, True),
    (2, 2, 1, 200, 64, False),
    (1, 2, 2, 640, 128, False),
    # causal grids that divide evenly over 8 XCDs with few row tiles per head: both
    # kernels take the rank-major workgroup order (longest tiles of several heads first)
    (2, 8, 8, 512, 128, True),
    (4, 8, 4, 1024, 128, True),
    (2, 8, 4, 512, 64, True),
])
def test_backward_full(B, H, Hkv, N, d, causal):
    note(f"backward full: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v, do = draw(B, H, Hkv, N, d, seed=B + H + Hkv + N + d + causal)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv, delta = run_gpu_backward(q, k, v, do, causal, scale)
    rq, rk, rv, rd = oracle.attention_backward(q, k, v, do, causal, scale)
    errs = [rel_err(dq, rq), rel_err(dk, rk), rel_err(dv, rv), rel_err(delta, rd)]
    note(f"  relative max errors dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e} D {errs[3]:.2e}")
    assert all(np.all(np.isfinite(x)) for x in (dq, dk, dv, delta))
    assert max(errs) <= TOL_REL, errs


@pytest.mark.parametrize("causal", [False, True])
def test_backward_headline_sampled(causal):
    """The headline shape (2 x 32 x 8192 x 128); sampled dQ rows of four heads and
    sampled dK/dV rows of two heads, normalised by the sampled reference's maximum."""
    B, H, N, d = 2, 32, 8192, 128
    note(f"backward sampled: B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v, do = draw(B, H, H, N, d, seed=2024 + causal)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv, delta = run_gpu_backward(q, k, v, do, causal, scale)
    rng = np.random.default_rng(5)
    rows = np.unique(np.r_[0, 1, 127, 128, 255, 256, 4095, 4096, N - 1, rng.integers(0, N, 40)])
    pq = [(0, 0, rows), (1, 31, rows), (0, 17, rows), (1, 5, rows)]
    pkv = [(0, 3, rows), (1, 30, rows)]
    rq, rkv = oracle.attention_backward_rows(q, k, v, do, causal, scale, pq, pkv)
    eq = max(rel_err(dq[b, h, r], x) for (b, h, r), x in zip(pq, rq))
    ek = max(rel_err(dk[b, g, r], xk) for (b, g, r), (xk, _) in zip(pkv, rkv))
    ev = max(rel_err(dv[b, g, r], xv) for (b, g, r), (_, xv) in zip(pkv, rkv))
    note(f"  sampled relative max errors dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
    assert max(eq, ek, ev) <= TOL_REL
    assert all(np.all(np.isfinite(x)) for x in (dq, dk, dv, delta))


def test_backward_gqa_equals_repeated_heads_summed():
    """Grouped K/V: dK and dV equal the multi-head gradients on repeated K/V heads,
    summed over each group, up to the bf16 rounding of the G = 4 per-head results
    (at most G * 2^-9 = 7.8e-3 of the largest; 1e-2 allowed)."""
    B, H, Hkv, N, d = 1, 8, 2, 384, 128
    q, k, v, do = draw(B, H, Hkv, N, d, seed=77)
    dq, dk, dv, _ = run_gpu_backward(q, k, v, do, True, 1 / math.sqrt(d))
    G = H // Hkv
    kr, vr = k.repeat_interleave(G, dim=1).contiguous(), v.repeat_interleave(G, dim=1).contiguous()
    dq2, dk2, dv2, _ = run_gpu_backward(q, kr, vr, do, True, 1 / math.sqrt(d))
    assert np.array_equal(dq, dq2)
    assert rel_err(dk, dk2.reshape(B, Hkv, G, N, d).sum(2)) <= 1e-2
    assert rel_err(dv, dv2.reshape(B, Hkv, G, N, d).sum(2)) <= 1e-2


def test_backward_deterministic():
    q, k, v, do = draw(1, 4, 2, 700, 128, seed=78)
    a = run_gpu_backward(q, k, v, do, True, 0.1)
    b = run_gpu_backward(q, k, v, do, True, 0.1)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_backward_wrapper_rejects_bad_tensors():
    dev = device()
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((1, 2, 64), dtype=torch.float32, device=dev)
    with pytest.raises(TypeError):
        binding.attention_backward(q, q, q, q, lse.double(), q)
    with pytest.raises(ValueError):
        binding.attention_backward(q, q, q, q[:, :, :32].contiguous(), lse, q)
    with pytest.raises(binding.AttnError):
        binding.attention_backward(q, q, q, q, lse, q, dq=q)  # output overlaps an input
