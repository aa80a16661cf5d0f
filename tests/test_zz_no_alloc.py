"""attn_fwd_splitkv_noalloc vs attn_fwd_splitkv through the C ABI (MI355X only).

The no-allocation entry point runs the split-key kernels on the library's device
scratch array instead of a caller workspace; with the same inputs, options and
unit split it must give the same results as attn_fwd_splitkv with a workspace,
bit for bit (same kernels, same workspace layout), and within the forward
tolerances of the fp64 oracle (max|O - O_ref| <= 2e-2, max|LSE - LSE_ref| <= 1e-3).
Two calls in a row, the second with a smaller input, check that the scratch kept
from the first call does not leak into the second. Sizes beyond the scratch array
are rejected on the host before any launch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import assert_close, device, note

pytestmark = pytest.mark.gpu


def both(q, k, v, causal, n_splits, out_dtype=torch.bfloat16):
    """(workspace result, no-allocation result) as CPU tensors."""
    dev = device()
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    B, H, N, d = q.shape
    o_ws, l_ws = binding.attention_splitkv(q, k, v, causal=causal, n_splits=n_splits, out_dtype=out_dtype)
    o_na = torch.full((B, H, N, d), float("nan"), dtype=out_dtype, device=dev)
    l_na = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    binding.attention_splitkv_noalloc(q, k, v, o_na, l_na, causal=causal, n_splits=n_splits)
    torch.cuda.synchronize()
    return (o_ws.cpu(), l_ws.cpu()), (o_na.cpu(), l_na.cpu())


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_workspace_entry_two_calls(causal):
    # first call: 2 heads x 3000 rows split 4 ways (the scratch holds 4 units of fp32
    # partials); second call: a smaller problem split 3 ways, whose units cover only
    # the start of the scratch the first call filled
    for (B, H, Hkv, N, d, n_splits, seed) in ((1, 2, 2, 3000, 128, 4, 501), (1, 2, 1, 700, 64, 3, 502)):
        note(f"noalloc: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} n_splits={n_splits}")
        q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=seed + causal)
        (o_ws, l_ws), (o_na, l_na) = both(q, k, v, causal, n_splits)
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), "O differs from attn_fwd_splitkv"
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), "LSE differs from attn_fwd_splitkv"
        o_ref, lse_ref = oracle.attention_gqa(q, k, v, causal, 1.0 / math.sqrt(d))
        assert_close(o_na.float().numpy().astype(np.float64), l_na.numpy().astype(np.float64), o_ref, lse_ref,
                     what="no-allocation split keys")


def test_noalloc_fp32_output_and_automatic_split():
    q, k, v = inputs.draw(1, 1, 5000, 128, seed=503)
    (o_ws, l_ws), (o_na, l_na) = both(q, k, v, True, 0, out_dtype=torch.float32)
    assert torch.equal(o_na.view(torch.int32), o_ws.view(torch.int32))
    assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32))


def test_noalloc_rejects_sizes_beyond_the_scratch():
    dev = device()
    B, H, N, d = 1, 16, 16384, 128
    need = binding.splitkv_workspace_size(B, H, N, d, 8)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, H, N), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(binding.AttnError) as e:
        binding.attention_splitkv_noalloc(q, q, q, out, lse, n_splits=8)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()), "a rejected call wrote its outputs"
