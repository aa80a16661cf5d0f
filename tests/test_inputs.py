"""Seeded workload generator: determinism and the stated structure (CPU only)."""
import math

import torch

from exact_attention_22_amd import inputs


def test_workloads_as_stated():
    shapes = [(w.B, w.H, w.N, w.d, w.causal, w.drift) for w in inputs.WORKLOADS]
    assert shapes == [(1, 2, 256, 64, False, False), (4, 16, 2048, 128, True, False),
                      (2, 32, 8192, 128, False, False), (1, 32, 32768, 128, True, False),
                      (2, 16, 8192, 64, True, True), (2, 32, 8192, 128, True, False)]
    assert [w.kv_heads for w in inputs.WORKLOADS] == [2, 16, 32, 32, 16, 8]
    for w in inputs.WORKLOADS:
        assert w.scale == torch.tensor(1 / math.sqrt(w.d), dtype=torch.float32).item()
    assert inputs.BY_NAME["headline"].flops == 4.0 * 2 * 32 * 8192 ** 2 * 128
    assert inputs.BY_NAME["long32k"].flops == 2.0 * 32 * 32768 ** 2 * 128


def test_deterministic_and_seed_sensitive():
    a = inputs.draw(1, 2, 64, 64, seed=5)
    b = inputs.draw(1, 2, 64, 64, seed=5)
    c = inputs.draw(1, 2, 64, 64, seed=6)
    assert inputs.digest(*a) == inputs.digest(*b) != inputs.digest(*c)
    assert all(t.dtype == torch.bfloat16 and t.is_contiguous() for t in a)


def test_bf16_is_round_to_nearest_of_fp32_draw():
    g = torch.Generator().manual_seed(9)
    q32 = torch.randn((1, 1, 16, 8), generator=g)
    q, _, _ = inputs.draw(1, 1, 16, 8, seed=9)
    assert torch.equal(q, q32.to(torch.bfloat16))


def test_drift_structure():
    """Key j carries 0.002*j*u and queries carry u, so q.k grows ~0.002*j along the keys."""
    d, N = 64, 4096
    q, k, v = inputs.draw(1, 1, N, d, seed=3, drift=True)
    q0, k0, _ = inputs.draw(1, 1, N, d, seed=3, drift=False)
    u = torch.full((d,), 1 / math.sqrt(d))
    proj = (k.float() - k0.float())[0, 0] @ u
    expect = 0.002 * torch.arange(N, dtype=torch.float32)
    assert torch.max(torch.abs(proj - expect)) < 0.02 + 0.004 * expect.max()
    assert torch.max(torch.abs((q.float() - q0.float())[0, 0] @ u - 1.0)) < 0.02


def test_value_magnitude_budget():
    """|V| stays under 8 so one bf16 half-ulp of O stays under the 2e-2 budget."""
    _, _, v = inputs.draw(2, 16, 8192, 64, seed=1005)
    assert v.float().abs().max().item() < 8.0


def test_gqa_draw_shapes_and_mha_case():
    q, k, v = inputs.draw_gqa(2, 8, 2, 16, 4, seed=11)
    assert q.shape == (2, 8, 16, 4) and k.shape == v.shape == (2, 2, 16, 4)
    a = inputs.draw_gqa(1, 3, 3, 16, 4, seed=12)
    b = inputs.draw(1, 3, 16, 4, seed=12)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
