"""Split-key attention on the HIP path vs the fp64 oracle (MI355X only).

The keys of every query tile are split into ranges computed by separate
workgroups and merged by log-sum-exp weights. The result is exact attention,
so the oracle is the definition (oracle.attention_gqa); tolerances as for the
other forward tests (max|O - O_ref| <= 2e-2, max|LSE - LSE_ref| <= 1e-3).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import assert_close, check_sampled, device, note, sample_picks

pytestmark = pytest.mark.gpu


def run_split(q, k, v, causal, scale, n_splits, **kw):
    dev = device()
    o, lse = binding.attention_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                                       n_splits=n_splits, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,n_splits", [
    (1, 2, 2, 1000, 128, False, 2),
    (1, 2, 2, 1000, 128, True, 3),
    (2, 4, 2, 700, 64, True, 5),
    (1, 2, 1, 2048, 128, False, 0),
    (1, 1, 1, 1, 64, True, 1),
    (1, 2, 2, 130, 128, True, 8),
    (1, 3, 3, 777, 64, False, 4),
])
def test_splitkv_full(B, H, Hkv, N, d, causal, n_splits):
    note(f"split keys: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} n_splits={n_splits}")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=N + H + n_splits + causal)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_split(q, k, v, causal, scale, n_splits)
    o_ref, lse_ref = oracle.attention_gqa(q, k, v, causal, scale)
    assert_close(o, lse, o_ref, lse_ref, what=f"split {n_splits}")


def test_splitkv_negative_scale_and_fp32_output():
    q, k, v = inputs.draw(1, 2, 600, 128, seed=91)
    o, lse = run_split(q, k, v, True, -0.09, 3, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.attention(q, k, v, True, -0.09)
    assert_close(o, lse, o_ref, lse_ref, what="negative scale, fp32 O")


def test_one_split_is_bitwise_the_plain_kernel():
    """One unit per query tile: the merge multiplies by exp(0) = 1, so O and LSE are
    bit for bit those of attn_fwd."""
    q, k, v = (t.to(device()) for t in inputs.draw(2, 4, 1500, 128, seed=92))
    for causal in (False, True):
        o1, l1 = binding.attention_splitkv(q, k, v, causal=causal, n_splits=1)
        o2, l2 = binding.attention(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 16384, 128, False), (1, 4, 32768, 128, True)])
def test_splitkv_low_occupancy_sampled(B, H, N, d, causal):
    """Shapes with fewer query tiles than compute units (automatic split count)."""
    note(f"split keys, low occupancy: B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = inputs.draw(B, H, N, d, seed=N + H)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_split(q, k, v, causal, scale, 0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    picks = sample_picks(B, H, N, seed=N, full_heads=((0, H - 1),))
    check_sampled(q, k, v, causal, scale, o, lse, picks, f"split B={B} H={H} N={N}")


def test_splitkv_rejects_bad_workspace():
    dev = device()
    q = torch.zeros((1, 2, 512, 128), dtype=torch.bfloat16, device=dev)
    need = binding.splitkv_workspace_size(1, 2, 512, 128, 2)
    small = torch.empty(need - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(binding.AttnError):
        binding.attention_splitkv(q, q, q, n_splits=2, workspace=small)
    with pytest.raises(binding.AttnError):
        binding.attention_splitkv(q, q, q, n_splits=2, workspace=q.view(torch.uint8).flatten())  # overlaps q
    # caught by the binding before the C call: wrong dtype, wrong device, not 1-D, fp32 out for bf16
    with pytest.raises(TypeError):
        binding.attention_splitkv(q, q, q, n_splits=2, workspace=torch.empty(need // 4, dtype=torch.float32,
                                                                             device=dev))
    with pytest.raises(ValueError):
        binding.attention_splitkv(q, q, q, n_splits=2, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        binding.attention_splitkv(q, q, q, n_splits=2, workspace=torch.empty((2, need), dtype=torch.uint8,
                                                                             device=dev))
    with pytest.raises(TypeError):
        binding.attention_splitkv(q, q, q, n_splits=2, out=torch.empty(q.shape, dtype=torch.float32, device=dev))
