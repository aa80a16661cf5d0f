"""HIP attention forward vs the fp64 CPU oracle, through the C ABI (MI355X only).

Tolerances: max|O - O_ref| <= 2e-2 and max|LSE - LSE_ref| <= 1e-3 for bf16 inputs
with fp32 accumulation. Inputs come from the seeded generator only; expected
values come from the oracle only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import (TOL_LSE, TOL_O, assert_close, check_sampled, device, max_err, note,
                            run_gpu, sample_picks)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("name", ["tiny", "causal2k"])
def test_workload_full(name):
    w = inputs.BY_NAME[name]
    note(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = inputs.workload_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention(q, k, v, w.causal, w.scale)
    assert_close(o, lse, o_ref, lse_ref, what=name)


@pytest.mark.parametrize("name", ["headline", "long32k", "drift8k"])
def test_workload_sampled(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    computes every row of one head and sampled rows (tile edges + 64 seeded) of all heads."""
    w = inputs.BY_NAME[name]
    note(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = inputs.workload_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    picks = sample_picks(w.B, w.H, w.N, seed=w.seed, full_heads=((w.B - 1, w.H - 1),))
    check_sampled(q, k, v, w.causal, w.scale, o, lse, picks, name)


# ---------------------------------------------------------------- persistent tile walk
# A launch has at most one workgroup per compute unit; each walks the query tiles
# of its XCD's range (causal: alternating direction every round). These shapes
# give several rounds per workgroup, a partial last round (even and odd, i.e.
# forward and reversed) and a partial last XCD range. O and LSE start as NaN, so a
# tile that no workgroup writes shows up as non-finite output.
@pytest.mark.parametrize("B,H,N,d,causal", [
    (2, 50, 2048, 64, True),     # 800 tiles, 100 per XCD: odd (reversed) partial last round
    (1, 101, 1792, 64, True),    # 707 tiles, 89 per XCD, last XCD range 84: even partial rounds
    (1, 101, 1792, 128, False),  # the same walk without the reversal
    (3, 7, 4096, 128, True),     # 336 tiles, 42 per XCD
])
def test_persistent_walk_shapes(B, H, N, d, causal):
    note(f"persistent walk: B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = inputs.draw(B, H, N, d, seed=B * 1000 + H + N + d + causal)
    scale = 1.0 / math.sqrt(d)
    dev = device()
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    binding.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_h = o.float().cpu().numpy().astype(np.float64)
    l_h = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(l_h)), "some query tile was not written"
    picks = sample_picks(B, H, N, seed=N + H, full_heads=((B - 1, H - 1),))
    check_sampled(q, k, v, causal, scale, o_h, l_h, picks, f"B={B} H={H} N={N} d={d} causal={causal}")


# ---------------------------------------------------------------- ragged / small shapes
SWEEP_N = [1, 2, 7, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_sweep(d, causal):
    for n in SWEEP_N:
        for (B, H) in ((1, 1), (2, 3)):
            q, k, v = inputs.draw(B, H, n, d, seed=n * 7 + d + causal)
            scale = 1.0 / math.sqrt(d)
            o, lse = run_gpu(q, k, v, causal, scale)
            o_ref, lse_ref = oracle.attention(q, k, v, causal, scale)
            assert_close(o, lse, o_ref, lse_ref, what=f"N={n} d={d} B={B} H={H} causal={causal}")


def test_empty_is_a_no_op():
    dev = device()
    q = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device=dev)
    o, lse = binding.attention(q, q, q, causal=True)
    assert o.shape == (2, 3, 0, 64) and lse.shape == (2, 3, 0)


# ---------------------------------------------------------------- special cases with closed forms
@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0_is_v0_bitwise(d):
    """Causal row 0 sees key 0 only: O0 = V0 exactly in bf16, LSE0 = scale*q0.k0."""
    q, k, v = inputs.draw(2, 4, 300, d, seed=31)
    dev = device()
    o, lse = binding.attention(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    ref = 0.125 * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert max_err(lse[:, :, 0].cpu().double().numpy(), ref.numpy()) <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_of_visible_values(causal):
    q, k, v = inputs.draw(1, 2, 200, 64, seed=32)
    o, lse = run_gpu(q, k, v, causal, 0.0)
    vv = v.double().numpy()
    n = np.arange(1, 201)
    mean = np.cumsum(vv, axis=2) / n[None, None, :, None] if causal else np.broadcast_to(vv.mean(2, keepdims=True), vv.shape)
    lref = np.broadcast_to(np.log(n) if causal else np.full(200, math.log(200)), lse.shape)
    assert_close(o, lse, mean, lref, what="scale=0")


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values(causal):
    q, k, _ = inputs.draw(1, 2, 333, 128, seed=33)
    row = inputs.draw(1, 1, 1, 128, seed=34)[2][0, 0, 0]
    v = row.expand(1, 2, 333, 128).contiguous()
    o, _ = run_gpu(q, k, v, causal, 1 / math.sqrt(128))
    assert max_err(o, np.broadcast_to(row.double().numpy(), o.shape)) <= TOL_O


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale(causal):
    q, k, v = inputs.draw(1, 2, 300, 64, seed=35)
    o, lse = run_gpu(q, k, v, causal, -0.2)
    o_ref, lse_ref = oracle.attention(q, k, v, causal, -0.2)
    assert_close(o, lse, o_ref, lse_ref, what="negative scale")


def test_large_logits_dominant_key():
    """A key far ahead of the rest: O tracks that key's value (exp range of the online softmax)."""
    q, k, v = inputs.draw(1, 1, 256, 64, seed=36)
    k = k.clone()
    k[0, 0, 77] = (q[0, 0].float().mean(0) * 0 + 4.0).to(torch.bfloat16)  # constant key row
    q = (q.float().abs() + 0.5).to(torch.bfloat16)   # positive queries: key 77 wins every row by a wide margin
    o, lse = run_gpu(q, k, v, False, 1.0)
    o_ref, lse_ref = oracle.attention(q, k, v, False, 1.0)
    assert_close(o, lse, o_ref, lse_ref, what="dominant key")


# ---------------------------------------------------------------- options
@pytest.mark.parametrize("tau", [0.0, 1.0, 2.0, 8.0, 64.0])
@pytest.mark.parametrize("poly", [0, 4, 8])
def test_rescale_threshold_and_exp2_split(tau, poly):
    """Any rescale threshold and any exp2 split reach the oracle (drifting logits, d=64 causal)."""
    q, k, v = inputs.draw(1, 4, 2048, 64, seed=1005, drift=True)
    scale = 0.125
    o, lse = run_gpu(q, k, v, True, scale, tau=tau, poly_eighths=poly)
    o_ref, lse_ref = oracle.attention(q, k, v, True, scale)
    assert_close(o, lse, o_ref, lse_ref, what=f"tau={tau} poly={poly}")


@pytest.mark.parametrize("d", [64, 128])
def test_adaptive_rescale_on_off_agree(d):
    """Adaptive (tau=8) and classic (tau=0) rescaling give the same result up to rounding (fp32 O)."""
    q, k, v = inputs.draw(2, 4, 1500, d, seed=40, drift=True)
    s = 1 / math.sqrt(d)
    o8, l8 = run_gpu(q, k, v, True, s, tau=8.0, out_dtype=torch.float32)
    o0, l0 = run_gpu(q, k, v, True, s, tau=0.0, out_dtype=torch.float32)
    note(f"  on/off: max|dO|={max_err(o8, o0):.2e} max|dLSE|={max_err(l8, l0):.2e}")
    assert max_err(o8, o0) <= 4e-3 and max_err(l8, l0) <= 1e-5
    o_ref, lse_ref = oracle.attention(q, k, v, True, s)
    assert_close(o8, l8, o_ref, lse_ref, tol_o=5e-3, what="fp32 O tau=8")


def test_fp32_output():
    q, k, v = inputs.draw(1, 3, 777, 128, seed=41)
    o, lse = run_gpu(q, k, v, False, 0.0884, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.attention(q, k, v, False, 0.0884)
    assert_close(o, lse, o_ref, lse_ref, tol_o=5e-3, what="fp32 O")


def test_rescale_counts_follow_the_threshold():
    """Instrumented rescale counts: tau=0 rescales on every increase, tau=8 almost never
    (the pages report about ten times fewer rescales with the adaptive policy). Per row the
    kernel's counts match the fp64 tiled model's with the same tiling; the kernel decides on
    fp32 scores and the model on fp64 ones, so only near-ties may differ (>= 99% must agree)."""
    q, k, v = inputs.draw(1, 2, 1024, 64, seed=1005, drift=True)
    s = 0.125
    _, _, c0 = run_gpu(q, k, v, True, s, tau=0.0, rescale_count=True)
    _, _, c8 = run_gpu(q, k, v, True, s, tau=8.0, rescale_count=True)
    note(f"  rescales: tau=0 {int(c0.sum())}  tau=8 {int(c8.sum())}")
    assert c0.sum() >= 10 * max(1, c8.sum())
    br, bc = binding.tile_shape(64)   # the model uses the kernel's tiling
    _, _, m0 = oracle.tiled_online_attention(q, k, v, True, s, br, bc, 0.0)
    agree = np.mean(c0 == m0)
    note(f"  per-row agreement with fp64 model (tau=0): {agree:.4f}")
    assert agree >= 0.99


# ---------------------------------------------------------------- determinism / structure
def test_bitwise_deterministic():
    q, k, v = inputs.draw(2, 8, 1024, 128, seed=50)
    dev = device()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = binding.attention(qd, kd, vd, causal=True)
    o2, l2 = binding.attention(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_heads_independent_and_prefix_consistent():
    """Each (b,h) equals a single-head run; causal rows < 256 equal a run truncated to 256 rows
    (same q-tile/kv-tile decomposition of those rows, so bitwise)."""
    q, k, v = inputs.draw(2, 3, 640, 64, seed=51)
    dev = device()
    o, l = binding.attention(q.to(dev), k.to(dev), v.to(dev), causal=True)
    o1, l1 = binding.attention(q[1:2, 2:3].contiguous().to(dev), k[1:2, 2:3].contiguous().to(dev),
                               v[1:2, 2:3].contiguous().to(dev), causal=True)
    ot, lt = binding.attention(q[:, :, :256].contiguous().to(dev), k[:, :, :256].contiguous().to(dev),
                               v[:, :, :256].contiguous().to(dev), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[1:2, 2:3], o1) and torch.equal(l[1:2, 2:3], l1)
    assert torch.equal(o[:, :, :256], ot) and torch.equal(l[:, :, :256], lt)


def test_writes_only_its_outputs():
    """Guard bands around O and LSE stay untouched (no out-of-bounds stores on a ragged shape)."""
    dev = device()
    q, k, v = inputs.draw(1, 2, 97, 128, seed=52)
    n_o, n_l = 1 * 2 * 97 * 128, 1 * 2 * 97
    obuf = torch.full((n_o + 4096,), 7.0, dtype=torch.bfloat16, device=dev)
    lbuf = torch.full((n_l + 1024,), 7.0, dtype=torch.float32, device=dev)
    o = obuf[2048:2048 + n_o].view(1, 2, 97, 128)
    lse = lbuf[512:512 + n_l].view(1, 2, 97)
    binding.attention(q.to(dev), k.to(dev), v.to(dev), causal=False, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:2048] == 7.0) and torch.all(obuf[2048 + n_o:] == 7.0)
    assert torch.all(lbuf[:512] == 7.0) and torch.all(lbuf[512 + n_l:] == 7.0)
    o_ref, l_ref = oracle.attention(q, k, v, False, 1 / math.sqrt(128))
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, what="guarded")


def test_python_wrapper_rejects_bad_outputs():
    """Caller-supplied out and lse are checked before the C call, which cannot see
    their size, dtype or device."""
    dev = device()
    q = torch.zeros((2, 3, 40, 64), dtype=torch.bfloat16, device=dev)
    bad_out = [
        (torch.empty(q.shape, dtype=torch.float32, device=dev), TypeError),        # fp32 O for bf16 out_dtype
        (torch.empty((2, 3, 39, 64), dtype=torch.bfloat16, device=dev), ValueError),  # undersized
        (torch.empty((2, 40, 3, 64), dtype=torch.bfloat16, device=dev).transpose(1, 2), ValueError),  # strided
        (torch.empty(q.shape, dtype=torch.bfloat16), ValueError),                  # host memory
    ]
    for out, exc in bad_out:
        with pytest.raises(exc):
            binding.attention(q, q, q, out=out)
    for lse, exc in [(torch.empty((2, 3, 40), dtype=torch.float64, device=dev), TypeError),
                     (torch.empty((2, 3, 20), dtype=torch.float32, device=dev), ValueError),
                     (torch.empty((2, 3, 40), dtype=torch.float32), ValueError)]:
        with pytest.raises(exc):
            binding.attention(q, q, q, lse=lse)
    with pytest.raises(TypeError):
        binding.attention(q, q, q, out_dtype=torch.float32, out=torch.empty(q.shape, dtype=torch.bfloat16, device=dev))
    # packed batches: [H, total, d] outputs
    qv = torch.zeros((3, 100, 64), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 60, 100], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        binding.attention_varlen(qv, qv, qv, cu, out=torch.empty((3, 99, 64), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        binding.attention_varlen(qv, qv, qv, cu, lse=torch.empty((3, 100), dtype=torch.float32))


def test_python_wrapper_rejects_bad_tensors():
    dev = device()
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(TypeError):
        binding.attention(q.float(), q, q)
    with pytest.raises(ValueError):
        binding.attention(q, q[:, :, :4], q)
    with pytest.raises(binding.AttnError):
        binding.attention(torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device=dev),
                          torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device=dev),
                          torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device=dev))
