"""Grouped-query and multi-query attention on the HIP path vs the fp64 oracle (MI355X only).

Query head h reads key/value head h // (H // Hkv) (consecutive groups; page
"FlashAttention 4: faster, more memory-efficient attention for LLMs", sections
"Key points" and "Compatibility and current status"). Tolerances as for the
multi-head tests: max|O - O_ref| <= 2e-2, max|LSE - LSE_ref| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import assert_close, check_sampled, device, note, run_gpu, sample_picks

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (1, 8, 2, 300, 64, False),
    (2, 8, 1, 513, 128, True),    # multi-query
    (1, 6, 3, 257, 128, True),
    (1, 4, 4, 200, 64, True),     # Hkv = H through the grouped entry point
    (1, 16, 2, 31, 128, False),   # shorter than one key tile
])
def test_gqa_full(B, H, Hkv, N, d, causal):
    note(f"gqa full: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=B + H + Hkv + N + d + causal)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_gpu(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention_gqa(q, k, v, causal, scale)
    assert_close(o, lse, o_ref, lse_ref, what=f"gqa B={B} H={H} Hkv={Hkv} N={N} d={d}")


def test_gqa_workload_sampled():
    """The full-size grouped-query workload (2 x 32 query heads, 8 key/value heads,
    N = 8192, d = 128, causal) in the benchmark's launch configuration."""
    w = inputs.BY_NAME["gqa8k"]
    note(f"workload gqa8k: B={w.B} H={w.H} Hkv={w.kv_heads} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = inputs.workload_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    picks = sample_picks(w.B, w.H, w.N, seed=w.seed, full_heads=((w.B - 1, w.H - 1), (0, 1)))
    check_sampled(q, k, v, w.causal, w.scale, o, lse, picks, "gqa8k")


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (2, 16, 4, 1024, 128, True),
    (1, 8, 1, 777, 64, False),
    (1, 12, 6, 1500, 64, True),
])
def test_gqa_bitwise_equals_mha_on_repeated_heads(B, H, Hkv, N, d, causal):
    """Grouped K/V give bit for bit the multi-head result on K/V whose heads are
    repeated to the query heads (each key/value head copied to its group)."""
    note(f"gqa vs repeated heads: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=7 * N + H)
    dev = device()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    G = H // Hkv
    kr = kd.repeat_interleave(G, dim=1).contiguous()
    vr = vd.repeat_interleave(G, dim=1).contiguous()
    o1, l1 = binding.attention(qd, kd, vd, causal=causal)
    o2, l2 = binding.attention(qd, kr, vr, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_entry_with_all_heads_is_attn_fwd_ex():
    B, H, N, d = 1, 4, 700, 128
    q, k, v = (t.to(device()) for t in inputs.draw(B, H, N, d, seed=41))
    scale = 1.0 / math.sqrt(d)
    outs = []
    for entry in ("ex", "gqa"):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        stream = torch.cuda.current_stream().cuda_stream
        if entry == "ex":
            st = binding.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, 1, scale, None, stream)
        else:
            st = binding.attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      B, H, H, N, d, 1, scale, None, stream)
        assert st == binding.ATTN_OK, binding.last_error()
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (3, 12, 4, 1792, 64, True),    # 252 tiles: the last XCD range is partial
    (2, 40, 5, 2304, 128, False),  # 720 tiles, 90 per XCD
])
def test_gqa_persistent_walk(B, H, Hkv, N, d, causal):
    note(f"gqa persistent walk: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=N + H + Hkv)
    scale = 1.0 / math.sqrt(d)
    dev = device()
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    binding.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_h = o.float().cpu().numpy().astype(np.float64)
    l_h = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(l_h)), "some query tile was not written"
    picks = sample_picks(B, H, N, seed=N + Hkv, full_heads=((B - 1, H - 1), (0, H // Hkv)))
    check_sampled(q, k, v, causal, scale, o_h, l_h, picks, f"gqa B={B} H={H} Hkv={Hkv} N={N} d={d}")


def test_gqa_wrapper_rejects_bad_shapes():
    dev = device()
    q = torch.zeros((1, 8, 64, 64), dtype=torch.bfloat16, device=dev)
    k3 = torch.zeros((1, 3, 64, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.AttnError):
        binding.attention(q, k3, k3)
    k2 = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device=dev)
    v4 = torch.zeros((1, 4, 64, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        binding.attention(q, k2, v4)
    k_short = torch.zeros((1, 2, 32, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        binding.attention(q, k_short, k_short)
