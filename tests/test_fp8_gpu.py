"""FP8 (e4m3) attention forward on the HIP path vs the fp64 oracle (MI355X only).

The oracle is exact attention of the dequantised codes (oracle.fp8). The
tolerance is the per-row bound oracle.fp8.fp8_error_bound derives from the
three roundings an FP8 kernel makes (the matrix core's e4m3 dot products, P
rounded to e4m3, O rounded to bf16): every row must satisfy
max_c |O_ic - O_ref,ic| <= bound_O,i and |LSE_i - LSE_ref,i| <= bound_LSE,i + 2e-5.
The observed errors are printed next to the bound.
"""
import numpy as np
import pytest
import torch

import oracle.fp8 as of
from exact_attention_22_amd import binding, inputs
from tests.gpu_util import device, note, sample_picks

pytestmark = pytest.mark.gpu

LSE_SLACK = 2e-5   # fp32 arithmetic of the row sum, exp2 and log2 (far below the bound's own size)


def run_fp8(q8, k8, vt8, sc, causal, scale, **kw):
    dev = device()
    o, lse = binding.attention_fp8(q8.to(dev), k8.to(dev), vt8.to(dev), sc, causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_rows(o, lse, o_ref, lse_ref, bo, bl, what):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    eo = np.abs(o - o_ref).max(axis=-1)
    el = np.abs(lse - lse_ref)
    note(f"  {what}: max|dO|={eo.max():.3e} (max ratio to bound {float((eo / bo).max()):.3f}) "
         f"max|dLSE|={el.max():.3e} (bound {float(bl.max()):.2e})")
    assert np.all(eo <= bo), f"{what}: O outside the bound in {int((eo > bo).sum())} rows"
    assert np.all(el <= bl + LSE_SLACK), f"{what}: LSE outside the bound"


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 256, 64, False),
    (1, 2, 256, 128, True),
    (2, 2, 200, 128, False),
    (1, 3, 77, 64, True),
    (1, 1, 1, 128, False),
    (1, 1, 17, 64, True),
    (1, 2, 1000, 128, True),
    (2, 1, 640, 64, False),
    # causal grids whose XCD ranges hold several whole heads of few query tiles: the
    # workgroups go by tile rank first (longest tiles of every head first)
    (2, 8, 512, 128, True),
    (4, 4, 512, 64, True),
])
def test_fp8_full(B, H, N, d, causal):
    note(f"fp8: B={B} H={H} N={N} d={d} causal={causal}")
    # padding columns of V^T hold NaN codes: the kernel must never read them
    q8, k8, vt8, sc = inputs.draw_fp8(B, H, N, d, seed=N + d + causal, pad_code=0x7F)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = run_fp8(q8, k8, vt8, sc, causal, scale)
    o_ref, lse_ref = of.attention_fp8(q8, k8, vt8, sc, causal, scale)
    bo, bl = of.fp8_error_bound(q8, k8, vt8, sc, causal, scale)
    check_rows(o, lse, o_ref, lse_ref, bo, bl, "fp8")


@pytest.mark.parametrize("tau", [0.0, 2.0, 8.0])
def test_fp8_rescale_thresholds_on_drift(tau):
    """Keys whose logits drift upwards keep raising the running maximum (rescale path)."""
    B, H, N, d = 1, 2, 1536, 64
    note(f"fp8 drift: tau={tau}")
    q8, k8, vt8, sc = inputs.draw_fp8(B, H, N, d, seed=1005, drift=True)
    scale = float(np.float32(0.125))
    o, lse = run_fp8(q8, k8, vt8, sc, True, scale, tau=tau)
    o_ref, lse_ref = of.attention_fp8(q8, k8, vt8, sc, True, scale)
    bo, bl = of.fp8_error_bound(q8, k8, vt8, sc, True, scale)
    check_rows(o, lse, o_ref, lse_ref, bo, bl, f"drift tau={tau}")


def test_fp8_causal_row0_is_v0():
    """Causal row 0 sees only key 0: P = 1 exactly, so O_0 = bf16(v_0 * v_scale) bit for bit."""
    q8, k8, vt8, sc = inputs.draw_fp8(2, 3, 300, 128, seed=77)
    o, lse = run_fp8(q8, k8, vt8, sc, True, 0.088)
    v0 = torch.from_numpy(of.e4m3_decode(vt8[..., 0].numpy())).float() * torch.tensor(sc[2], dtype=torch.float32)
    assert np.array_equal(o[:, :, 0], v0.to(torch.bfloat16).double().numpy())


def test_fp8_deterministic():
    q8, k8, vt8, sc = inputs.draw_fp8(1, 4, 999, 128, seed=5)
    a = run_fp8(q8, k8, vt8, sc, True, 0.09)
    b = run_fp8(q8, k8, vt8, sc, True, 0.09)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_headline_sampled():
    """Full headline shape 2 x 32 x 8192 x 128, non-causal, in the launch configuration the
    benchmark times; sampled rows against the oracle."""
    w = inputs.FP8_HEADLINE
    note(f"fp8 headline {w.B}x{w.H}x{w.N}x{w.d}")
    q8, k8, vt8, sc = inputs.draw_fp8(w.B, w.H, w.N, w.d, seed=w.seed)
    o, lse = run_fp8(q8, k8, vt8, sc, w.causal, w.scale)
    picks = sample_picks(w.B, w.H, w.N, seed=7, full_heads=())
    refs = of.attention_fp8_rows(q8, k8, vt8, sc, w.causal, w.scale, picks)
    bounds = of.fp8_error_bound_rows(q8, k8, vt8, sc, w.causal, w.scale, picks)
    eo_all, ratio = 0.0, 0.0
    for (b, h, rows), (o_ref, l_ref), (bo, bl) in zip(picks, refs, bounds):
        eo = np.abs(o[b, h, rows] - o_ref).max(axis=-1)
        el = np.abs(lse[b, h, rows] - l_ref)
        assert np.all(eo <= bo) and np.all(el <= bl + LSE_SLACK), (b, h)
        eo_all, ratio = max(eo_all, float(eo.max())), max(ratio, float((eo / bo).max()))
    note(f"  sampled {sum(len(r) for _, _, r in picks)} rows: max|dO|={eo_all:.3e} (ratio to bound {ratio:.3f})")


def test_fp8_causal_long_sampled():
    """Causal 1 x 8 x 8192 x 128 (the long-context shape at fewer heads)."""
    q8, k8, vt8, sc = inputs.draw_fp8(1, 8, 8192, 128, seed=1004)
    scale = float(np.float32(1 / np.sqrt(128)))
    o, lse = run_fp8(q8, k8, vt8, sc, True, scale)
    picks = sample_picks(1, 8, 8192, seed=9, full_heads=())
    refs = of.attention_fp8_rows(q8, k8, vt8, sc, True, scale, picks)
    bounds = of.fp8_error_bound_rows(q8, k8, vt8, sc, True, scale, picks)
    for (b, h, rows), (o_ref, l_ref), (bo, bl) in zip(picks, refs, bounds):
        eo = np.abs(o[b, h, rows] - o_ref).max(axis=-1)
        el = np.abs(lse[b, h, rows] - l_ref)
        assert np.all(eo <= bo) and np.all(el <= bl + LSE_SLACK), (b, h)


def test_fp8_wrapper_rejects_bad_arguments():
    dev = device()
    q8, k8, vt8, sc = inputs.draw_fp8(1, 1, 40, 64, seed=1)
    q, k, vt = q8.to(dev), k8.to(dev), vt8.to(dev)
    with pytest.raises(ValueError):
        binding.attention_fp8(q, k, vt[..., :40].contiguous(), sc)
    with pytest.raises(binding.AttnError):
        binding.attention_fp8(q, k, vt, sc, tau=9.0)
    with pytest.raises(binding.AttnError):
        binding.attention_fp8(q, k, vt, (0.0, 1.0, 1.0))


def test_fp8_wide_range_codes_stay_within_dot_product_bound():
    """Q and K codes drawn uniformly over every finite e4m3 value (magnitudes 2^-9 .. 448, the
    worst case for the alignment inside the matrix instruction): the LSE error must stay within
    the score bound E = 2^-10 * scale * max_j sum_k |q_k k_k| that the oracle assumes for the
    matrix core's e4m3 dot products, and O within its per-row bound."""
    B, H, N, d = 1, 2, 384, 128
    g = torch.Generator().manual_seed(123)
    codes = torch.randint(0, 256, (3, B, H, N, d), generator=g, dtype=torch.int32).to(torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38      # NaN patterns -> 1.0
    q8, k8, v8 = codes[0].contiguous(), codes[1].contiguous(), codes[2]
    vt8 = torch.zeros((B, H, d, inputs.fp8_ldv(N)), dtype=torch.uint8)
    vt8[..., :N] = v8.transpose(-1, -2)
    sc = (1.0 / 448, 1.0 / 448, 1.0 / 448)
    for causal in (False, True):
        o, lse = run_fp8(q8, k8, vt8, sc, causal, 0.5)
        o_ref, lse_ref = of.attention_fp8(q8, k8, vt8, sc, causal, 0.5)
        bo, bl = of.fp8_error_bound(q8, k8, vt8, sc, causal, 0.5)
        check_rows(o, lse, o_ref, lse_ref, bo, bl, f"wide-range codes causal={causal}")
