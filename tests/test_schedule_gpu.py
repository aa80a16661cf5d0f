"""Race check of the pipelined kernels (MI355X only).

Each kernel has a reference schedule (attn_fwd_opts.schedule = 1, attn_fwd_fp8_ex
with schedule 1) that computes the same tiles with the same instructions in the
same order, but loads every tile into LDS between two block-wide barriers and
reads it only after the second: nothing is in flight while anything is read. The
pipelined schedule overlaps the loads of later tiles with the products of the
current one across double buffers and two groups of wavefronts. If one of its
waits or barriers were missing or misplaced, some wavefront would read a tile
before it landed or after it was overwritten, and its result would differ from
the reference schedule's in some element; the two must therefore agree BITWISE,
in O and in LSE.

The shapes cover each way the pipeline walks its tiles: the persistent walk (more
query tiles than compute units, so each workgroup issues the next tile's loads
during this tile's epilogue), ragged key tails, causal diagonals, grouped-query
heads, packed variable-length sequences (including sequences shorter than one key
tile) and split keys; the drifting inputs and tau = 0 make rows rescale often, so
the rescale branch runs between loads. The FP8 kernel is checked the same way, and
the backward's wavefront-pair dk/dv kernel against the one-wavefront kernel.
"""
import math

import pytest
import torch

from exact_attention_22_amd import binding, inputs
from tests.gpu_util import device, note

pytestmark = pytest.mark.gpu

REF = binding.SCHEDULE_REFERENCE


def same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    assert a.dtype == b.dtype and a.shape == b.shape
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    diff = int((ia != ib).sum())
    note(f"  {what}: {a.numel()} elements, {diff} differ")
    assert diff == 0, f"{what}: {diff} of {a.numel()} elements differ between the schedules"


def tiles_and_cus(B, H, N, d):
    rows, _ = binding.tile_shape(d)
    return B * H * ((N + rows - 1) // rows), torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,drift,tau,f32", [
    (2, 16, 16, 4096, 128, False, False, 8.0, False),  # persistent walk, full tiles
    (2, 16, 16, 4000, 128, True, True, 8.0, False),    # persistent walk, causal, ragged tail, rescales
    (1, 24, 24, 3001, 64, False, True, 0.0, True),     # d = 64, classic rescale policy, fp32 O
    (2, 20, 20, 4097, 64, True, False, 8.0, False),    # d = 64 persistent walk, one-key tail tile
    (1, 16, 4, 2500, 128, True, True, 8.0, False),     # grouped-query heads
    (2, 32, 8, 1000, 64, False, False, 8.0, True),     # grouped-query heads, d = 64
    (1, 2, 2, 37, 128, False, False, 8.0, False),      # shorter than one key tile
])
def test_dense_and_gqa_schedules_agree_bitwise(B, H, Hkv, N, d, causal, drift, tau, f32):
    tiles, cus = tiles_and_cus(B, H, N, d)
    note(f"schedules dense: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} drift={drift} tau={tau} "
         f"fp32 O={f32} ({tiles} query tiles, {cus} compute units)")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=31000 + N + d + H, drift=drift)
    dev = device()
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    dt = torch.float32 if f32 else torch.bfloat16
    o1, l1 = binding.attention(q, k, v, causal=causal, tau=tau, out_dtype=dt)
    o2, l2 = binding.attention(q, k, v, causal=causal, tau=tau, out_dtype=dt, schedule=REF)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    same_bits(o1, o2, "O")
    same_bits(l1, l2, "LSE")


def test_persistent_walk_shapes_really_walk():
    # the first dense cases must launch fewer workgroups than query tiles
    for (B, H, N, d) in ((2, 16, 4096, 128), (2, 16, 4000, 128), (2, 20, 4097, 64)):
        tiles, cus = tiles_and_cus(B, H, N, d)
        assert tiles > cus, (B, H, N, d, tiles, cus)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_schedules_agree_bitwise(d, causal):
    lengths = [1, 63, 64, 65, 0, 1000, 2500, 17, 640, 129] + inputs.varlen_lengths(40, 16, 3000, seed=77 + d)
    H, Hkv = 8, 2
    note(f"schedules varlen: {len(lengths)} sequences, total {sum(lengths)}, H={H} Hkv={Hkv} d={d} causal={causal}")
    q, k, v, cu = inputs.draw_varlen(lengths, H, Hkv, d, seed=32000 + d + causal)
    dev = device()
    q, k, v, cu = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    o1, l1 = binding.attention_varlen(q, k, v, cu, causal=causal)
    o2, l2 = binding.attention_varlen(q, k, v, cu, causal=causal, schedule=REF)
    torch.cuda.synchronize()
    same_bits(o1, o2, "O")
    same_bits(l1, l2, "LSE")


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,splits", [
    (1, 4, 4, 8192, 128, False, 4),
    (1, 4, 2, 8000, 128, True, 3),
    (1, 2, 2, 16384, 64, False, 0),   # automatic split count
    (2, 3, 3, 5001, 64, True, 5),
])
def test_splitkv_schedules_agree_bitwise(B, H, Hkv, N, d, causal, splits):
    note(f"schedules split keys: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} n_splits={splits}")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=33000 + N + d, drift=True)
    dev = device()
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = binding.attention_splitkv(q, k, v, causal=causal, n_splits=splits)
    o2, l2 = binding.attention_splitkv(q, k, v, causal=causal, n_splits=splits, schedule=REF)
    torch.cuda.synchronize()
    same_bits(o1, o2, "O")
    same_bits(l1, l2, "LSE")


@pytest.mark.parametrize("B,H,N,d,causal,drift,tau", [
    (2, 16, 4096, 128, False, False, 8.0),
    (1, 8, 3001, 128, True, True, 0.0),
    (2, 8, 2049, 64, False, True, 8.0),
    (1, 4, 700, 64, True, False, 4.0),
    (1, 2, 40, 128, False, False, 8.0),
])
def test_fp8_schedules_agree_bitwise(B, H, N, d, causal, drift, tau):
    note(f"schedules fp8: B={B} H={H} N={N} d={d} causal={causal} drift={drift} tau={tau}")
    q8, k8, vt8, sc = inputs.draw_fp8(B, H, N, d, seed=34000 + N + d, drift=drift, pad_code=0x7F)
    dev = device()
    q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
    scale = 1.0 / math.sqrt(d)
    o1, l1 = binding.attention_fp8(q8, k8, vt8, sc, causal=causal, scale=scale, tau=tau)
    o2, l2 = binding.attention_fp8(q8, k8, vt8, sc, causal=causal, scale=scale, tau=tau, schedule=REF)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    same_bits(o1, o2, "O")
    same_bits(l1, l2, "LSE")


# Backward at d = 128: the dk/dv kernel runs in wavefront pairs that pass P through
# LDS (one wavefront forms S, P and dV, the other dP, dS and dK, with the tile loads
# issued by the second); the reference schedule computes dK and dV with the
# one-wavefront kernel, which keeps P in its lanes and accumulates every product in
# the same order. A missing or misplaced wait around the P buffer, the LSE tile or
# the tile loads would change some element of dK or dV. (d = 64 runs the
# one-wavefront kernel either way; one shape checks that the option is accepted.)
@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (2, 8, 8, 1024, 128, False),   # several query tiles per key block, full tiles
    (1, 8, 2, 1000, 128, True),    # grouped-query heads (4 per K/V head), causal, ragged
    (1, 4, 1, 777, 128, True),     # multi-query, causal, ragged
    (1, 4, 4, 37, 128, False),     # shorter than one tile
    (2, 4, 4, 513, 64, True),      # d = 64
])
def test_backward_schedules_agree_bitwise(B, H, Hkv, N, d, causal):
    note(f"schedules backward: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = inputs.draw_gqa(B, H, Hkv, N, d, seed=36000 + N + d + H)
    do = inputs.draw(B, H, N, d, seed=36500 + N)[0]
    dev = device()
    q, k, v, do = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    scale = 1.0 / math.sqrt(d)
    o, lse = binding.attention(q, k, v, causal=causal, scale=scale)
    g1 = binding.attention_backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    g2 = binding.attention_backward(q, k, v, o, lse, do, causal=causal, scale=scale, schedule=REF)
    torch.cuda.synchronize()
    for x in g1:
        assert torch.isfinite(x.float()).all()
    for name, a, b in zip(("dQ", "dK", "dV", "delta"), g1, g2):
        same_bits(a, b, name)


def test_reference_schedule_rejects_what_it_does_not_cover():
    dev = device()
    q, k, v = (t.to(dev) for t in inputs.draw(1, 1, 64, 64, seed=35000))
    with pytest.raises(binding.AttnError, match="ATTN_ERR_UNSUPPORTED"):
        binding.attention(q, k, v, poly_eighths=4, schedule=REF)
    with pytest.raises(binding.AttnError, match="ATTN_ERR_UNSUPPORTED"):
        binding.attention(q, k, v, scale=-0.125, schedule=REF)
    with pytest.raises(binding.AttnError, match="ATTN_ERR_OPTS"):
        binding.attention(q, k, v, schedule=2)
    o, lse = binding.attention(q, k, v)
    with pytest.raises(binding.AttnError, match="ATTN_ERR_OPTS"):
        binding.attention_backward(q, k, v, o, lse, q, schedule=2)
