"""Packed variable-length batches on the HIP path vs the fp64 oracle (MI355X only).

Layout: q, o [H,total,d], k, v [Hkv,total,d], lse [H,total]; sequence b is
tokens cu[b] .. cu[b+1]-1 (page "FlashAttention 4: faster, more memory-efficient
attention for LLMs", section "Key points"). Tolerances as for the dense tests:
max|O - O_ref| <= 2e-2, max|LSE - LSE_ref| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, device, max_err, note

pytestmark = pytest.mark.gpu


def run_varlen(q, k, v, cu, causal, scale, max_seqlen=None, fill_nan=False, **kw):
    dev = device()
    H, T, d = q.shape
    out = lse = None
    if fill_nan:
        out = torch.full((H, T, d), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev)
    res = binding.attention_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max_seqlen, causal=causal,
                                   scale=scale, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return res[0].float().cpu().numpy().astype(np.float64), res[1].cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths,H,Hkv", [
    ([300, 1, 0, 513, 256, 77], 4, 2),
    ([0, 5, 0], 2, 1),
    ([1000], 2, 2),
    ([64, 255, 257, 31, 32, 33, 128], 3, 1),
])
def test_varlen_full(lengths, H, Hkv, d, causal):
    note(f"varlen full: lengths={lengths} H={H} Hkv={Hkv} d={d} causal={causal}")
    q, k, v, cu = inputs.draw_varlen(lengths, H, Hkv, d, seed=sum(lengths) + H + d + causal)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_varlen(q, k, v, cu, causal, scale, fill_nan=True)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu, causal, scale)
    assert_close(o, lse, o_ref, lse_ref, what=f"varlen {lengths} d={d}")


def _boundary_picks(cu, H, seed, per_head=48):
    """Every head: the first two and last two tokens of every sequence, plus seeded tokens."""
    rng = np.random.default_rng(seed)
    cu = cu.tolist()
    edges = set()
    for a, e in zip(cu[:-1], cu[1:]):
        for t in (a, a + 1, e - 2, e - 1, a + 255, a + 256):
            if a <= t < e:
                edges.add(t)
    picks = []
    for h in range(H):
        toks = sorted(edges | set(rng.integers(0, cu[-1], per_head).tolist()))
        picks.append((h, np.asarray(toks)))
    return picks


def test_varlen_workload_sampled():
    """The packed workload (24 sequences of 64..8192 tokens, 32 query heads, 8 key/value
    heads, d = 128, causal) in the benchmark's launch configuration; every token of
    the longest sequence of head 5, and sequence edges plus seeded tokens of every head."""
    w = inputs.VARLEN
    note(f"workload varlen: lengths={w.lengths} H={w.H} Hkv={w.Hkv} d={w.d}")
    q, k, v, cu = w.inputs()
    o, lse = run_varlen(q, k, v, cu, w.causal, w.scale, fill_nan=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "some row was not written"
    picks = _boundary_picks(cu, w.H, seed=w.seed)
    b = int(np.argmax(w.lengths))
    picks.append((5, np.arange(int(cu[b]), int(cu[b + 1]))))
    refs = oracle.attention_varlen_rows(q, k, v, cu, w.causal, w.scale, picks)
    eo = el = 0.0
    for (h, toks), (o_ref, l_ref) in zip(picks, refs):
        eo = max(eo, max_err(o[h, toks], o_ref))
        el = max(el, max_err(lse[h, toks], l_ref))
    note(f"  varlen: {sum(len(t) for _, t in picks)} sampled rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (1, 4, 2, 1500, 128, True),
    (3, 8, 8, 512, 64, False),
    (4, 6, 3, 700, 128, True),
])
def test_equal_lengths_bitwise_equal_dense(B, H, Hkv, N, d, causal):
    """B sequences of one length N, packed, give bit for bit the dense [B,H,N,d] result."""
    note(f"varlen vs dense: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v, cu = inputs.draw_varlen([N] * B, H, Hkv, d, seed=B * N + H)
    dev = device()
    o1, l1 = binding.attention_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), causal=causal)
    dense = [t.view(t.shape[0], B, N, d).permute(1, 0, 2, 3).contiguous().to(dev) for t in (q, k, v)]
    o2, l2 = binding.attention(*dense, causal=causal)
    torch.cuda.synchronize()
    o2p = o2.permute(1, 0, 2, 3).reshape(H, B * N, d)
    l2p = l2.permute(1, 0, 2).reshape(H, B * N)
    assert torch.equal(o1, o2p) and torch.equal(l1, l2p)


def test_short_max_seqlen_leaves_later_rows_unwritten():
    """max_seqlen = 256 with a 600-token sequence: its first 256 rows are computed
    (over all its keys) and the rest keep their old contents; the other sequence is whole."""
    lengths, H, d = [600, 100], 2, 64
    q, k, v, cu = inputs.draw_varlen(lengths, H, H, d, seed=61)
    for causal in (False, True):
        o, lse = run_varlen(q, k, v, cu, causal, 0.125, max_seqlen=256, fill_nan=True)
        o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu, causal, 0.125)
        done = np.r_[0:256, 600:700]
        assert_close(o[:, done], lse[:, done], o_ref[:, done], lse_ref[:, done], what=f"computed rows causal={causal}")
        assert np.all(np.isnan(o[:, 256:600])) and np.all(np.isnan(lse[:, 256:600]))


def test_varlen_rescale_counts_and_fp32_output():
    q, k, v, cu = inputs.draw_varlen([700, 90, 1200], 2, 1, 128, seed=62)
    dev = device()
    o32, l32, cnt = binding.attention_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), causal=True,
                                             out_dtype=torch.float32, rescale_count=True, tau=0.0)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32 and cnt.shape == (2, 1990)
    assert int(cnt.min()) >= 0 and int(cnt.max()) <= 1200 // 64
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu, True, 1.0 / math.sqrt(128))
    assert_close(o32.cpu().double().numpy(), l32.cpu().double().numpy(), o_ref, lse_ref, what="fp32 O")


def test_varlen_deterministic():
    q, k, v, cu = inputs.draw_varlen([513, 1024, 7], 4, 2, 128, seed=63)
    dev = device()
    args = [t.to(dev) for t in (q, k, v, cu)]
    a = binding.attention_varlen(*args, causal=True)
    b = binding.attention_varlen(*args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_wrapper_rejects_bad_arguments():
    dev = device()
    q = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 30, 64], dtype=torch.int32, device=dev)
    with pytest.raises(TypeError):
        binding.attention_varlen(q, kv, kv, cu.long())
    with pytest.raises(TypeError):
        binding.attention_varlen(q, kv, kv, cu.cpu())
    with pytest.raises(ValueError):
        binding.attention_varlen(q, kv[:, :32], kv[:, :32], cu)
    with pytest.raises(binding.AttnError):
        binding.attention_varlen(q, kv[:3].repeat(2, 1, 1)[:3].contiguous(), kv[:3].repeat(2, 1, 1)[:3].contiguous(), cu)
