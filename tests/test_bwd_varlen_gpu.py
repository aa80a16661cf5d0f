"""Backward of packed variable-length attention on the HIP path vs the fp64 oracle (MI355X only).

The GPU forward (attn_fwd_varlen) supplies O and LSE; the oracle
(oracle.attention_backward_varlen) computes dQ, dK, dV and D from q, k, v and dO
alone. Tolerance as for the dense backward (tests/test_bwd_gpu.py, derived in its
header): max|X - X_ref| <= 2e-2 * max|X_ref| per tensor.
"""
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


def draw(lengths, H, Hkv, d, seed):
    q, k, v, cu = inputs.draw_varlen(lengths, H, Hkv, d, seed)
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do, cu


def run(q, k, v, do, cu, causal, scale, max_seqlen=None):
    dev = device()
    qd, kd, vd, dod, cud = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = binding.attention_varlen(qd, kd, vd, cud, max_seqlen=max_seqlen, causal=causal, scale=scale)
    grads = binding.attention_backward_varlen(qd, kd, vd, o, lse, dod, cud, max_seqlen=max_seqlen, causal=causal,
                                              scale=scale)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in grads)


@pytest.mark.parametrize("lengths", [[300, 1, 0, 513, 256, 77], [0, 5, 0], [1000], [64, 255, 257, 31, 32, 33, 128]])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_full(lengths, d, causal):
    H, Hkv = 4, 2
    note(f"varlen backward: lengths={lengths} H={H} Hkv={Hkv} d={d} causal={causal}")
    q, k, v, do, cu = draw(lengths, H, Hkv, d, seed=sum(lengths) + d + causal)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    got = run(q, k, v, do, cu, causal, scale)
    refs = oracle.attention_backward_varlen(q, k, v, do, cu.numpy(), causal, scale)
    errs = [rel_err(x, r) for x, r in zip(got, refs)]
    note(f"  relative max errors dQ dK dV D: {['%.2e' % e for e in errs]}")
    assert all(np.isfinite(x).all() for x in got)
    assert max(errs) <= TOL_REL, errs


def test_bwd_varlen_equal_lengths_match_dense_bitwise():
    """B sequences of one length N packed: the same bits as the dense backward on [B,H,N,d]."""
    B, H, Hkv, N, d = 3, 4, 2, 200, 128
    q, k, v, do, cu = draw([N] * B, H, Hkv, d, seed=3)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    dev = device()
    for causal in (False, True):
        got = run(q, k, v, do, cu, causal, scale)

        def dense(t, heads):  # [heads, B*N, d] -> [B, heads, N, d]
            return t.view(heads, B, N, d).transpose(0, 1).contiguous().to(dev)
        qd, kd, vd, dod = dense(q, H), dense(k, Hkv), dense(v, Hkv), dense(do, H)
        o, lse = binding.attention(qd, kd, vd, causal=causal, scale=scale)
        dq, dk, dv, delta = binding.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
        torch.cuda.synchronize()

        def packed(t, heads):  # [B, heads, N, d] -> [heads, B*N, d]
            return t.transpose(0, 1).reshape(heads, B * N, -1).float().cpu().numpy().astype(np.float64)
        ref = (packed(dq, H), packed(dk, Hkv), packed(dv, Hkv), packed(delta.unsqueeze(-1), H)[..., 0])
        for x, r, name in zip(got, ref, ("dq", "dk", "dv", "delta")):
            assert np.array_equal(x, r), f"{name} differs (causal={causal})"


def test_bwd_varlen_workload_sampled():
    """The varlen workload's lengths (24 sequences, 80..5753 tokens) at 8 query / 2 key-value
    heads: every gradient of the three shortest and the longest sequence against the oracle."""
    w = inputs.VARLEN
    lengths = w.lengths
    H, Hkv = 8, 2
    q, k, v, do, cu = draw(lengths, H, Hkv, w.d, seed=w.seed)
    got = run(q, k, v, do, cu, True, w.scale)
    cun = cu.numpy()
    order = np.argsort(lengths)
    for s in list(order[:3]) + [order[-1]]:
        a, e = int(cun[s]), int(cun[s + 1])
        refs = oracle.attention_backward(q[:, a:e].unsqueeze(0), k[:, a:e].unsqueeze(0), v[:, a:e].unsqueeze(0),
                                         do[:, a:e].unsqueeze(0), True, w.scale)
        errs = [rel_err(x[:, a:e], r[0]) for x, r in zip(got, refs)]
        note(f"  sequence {s} ({e - a} tokens): {['%.2e' % x for x in errs]}")
        assert max(errs) <= TOL_REL, (s, errs)


def test_bwd_varlen_wrapper_rejects_bad_arguments():
    dev = device()
    q, k, v, do, cu = draw([10, 20], 2, 1, 64, seed=1)
    qd, kd, vd, dod, cud = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = binding.attention_varlen(qd, kd, vd, cud)
    with pytest.raises(TypeError):
        binding.attention_backward_varlen(qd, kd, vd, o, lse, dod, cu)            # cu_seqlens on the host
    with pytest.raises(ValueError):
        binding.attention_backward_varlen(qd, kd, vd, o, lse, dod[:, :5].contiguous(), cud)
    with pytest.raises(binding.AttnError):
        binding.attention_backward_varlen(qd, kd, vd, o, lse, dod, cud, max_seqlen=-1)
