"""Exactness-isolating GPU tests: inputs chosen so that every product and sum the
HIP path forms is exact, leaving only the roundings the method itself takes
(MI355X only). Each test derives its bound below and checks every element of O
and LSE against the fp64 oracle; the bounds are several times tighter than the
general forward tolerances (2e-2, 1e-3), so a slip of a few thousandths in the
softmax stage fails them.

bf16 (the forward kernel). Q and K entries are multiples of 1/4 in [-2, 2] and V
entries multiples of 1/8 in [-1, 1], all exact in bf16.
  * S = Q K^T is exact in fp32: every product is a multiple of 1/16 of magnitude
    <= 4, every partial sum a multiple of 1/16 of magnitude <= 4d <= 512, i.e. at
    most 14 significant bits, whatever the order of accumulation.
  * x = s*c - m (one fma, c = fp32(scale) * fp32(log2 e)) and v_exp_f32 give P with
    relative error below 1e-5 (|s*c| <= 512 * 0.18 = 92 in log2 units, three fp32
    roundings of c and x; the exponential is within a few ulp).
  * P is rounded to bf16 (8 significant bits, round to nearest even): relative
    error <= 2^-8. The row sum l takes the unrounded fp32 P, so
    |O - O_exact| <= sum_j |bf16(P_j) - P_j| |v_j| / l <= 2^-8 max|v| = 2^-8.
  * P V accumulates exact bf16 x bf16 products in fp32 over <= N = 1000 terms:
    <= N 2^-24 max|v| = 6e-5; the normalisation O = acc * (1/l) adds two fp32
    roundings.
  * bf16 O: |O| <= 1 rounds with error <= 2^-9; fp32 O adds nothing visible.
  Bound: 2^-8 + 2^-9 + 1e-4 = 5.96e-3 (bf16 O) and 2^-8 + 1e-4 = 4.0e-3 (fp32 O).
  LSE = ln 2 (m + log2 l) with l from fp32 P: relative error of l below 2e-5, and
  the scale factor error shifts LSE by at most 3 2^-24 |scale s| <= 2e-5: 5e-5.

FP8 (attn_fwd_fp8). Q rows hold exactly nine 1.0 codes (0x38) at seeded
positions, zeros elsewhere; K codes are 0 or 1.0; V codes are 0, +-0.5, +-1;
all dequantisation scales 1 and scale = fp32(ln 2), so c = scale * log2 e rounds
to exactly 1.0 in fp32.
  * Every score s = |Q_i & K_j| is an integer in [0, 9], exact whatever the matrix
    core's internal alignment (integers below 2^4).
  * With tau = 0 the maximum in use is the running maximum, so x - m is an integer
    in [-9, 0]: P = 2^(x - m) is exact in fp32 and in e4m3 (2^-9 is its smallest
    subnormal), and every rescale factor is an exact power of two.
  * P V: products are 0 or powers of two in [2^-10, 1], every partial sum a
    multiple of 2^-10 below N = 1000: at most 20 significant bits, exact. The row
    sum is exact for the same reason.
  * Only O = acc * (1/l) (two fp32 roundings) and the bf16 rounding of O remain:
    |O - O_ref| <= 2^-8 |O_ref| + 1e-5 per element (the absolute part covers fp32
    roundings of sums that a rescale by 2^-k pushed below 2^-9); LSE = ln 2 (m + log2 l) with
    m exact and l within a few fp32 roundings: |LSE - LSE_ref| <= 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of
from exact_attention_22_amd import binding
from tests.gpu_util import device, max_err, note

pytestmark = pytest.mark.gpu

N_ROWS = 1000  # several 256-row query tiles and 64-key tiles, with ragged tails


def dyadic(shape, step, lim, seed):
    g = torch.Generator().manual_seed(seed)
    n = int(round(lim / step))
    return (torch.randint(-n, n + 1, shape, generator=g).float() * step).to(torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("out_f32,tau", [(False, 8.0), (True, 8.0), (False, 0.0)])
def test_dyadic_grid_isolates_the_softmax_stage(d, causal, out_f32, tau):
    note(f"dyadic grid: d={d} causal={causal} fp32 O={out_f32} tau={tau}")
    B, H, N = 1, 2, N_ROWS
    seed = 7000 + d + 10 * causal + 100 * out_f32 + int(tau)
    q = dyadic((B, H, N, d), 0.25, 2.0, seed)
    k = dyadic((B, H, N, d), 0.25, 2.0, seed + 1)
    v = dyadic((B, H, N, d), 0.125, 1.0, seed + 2)
    assert torch.equal(q.float().to(torch.bfloat16), q)  # grid values are exact in bf16
    scale = float(np.float32(1.0 / math.sqrt(d)))
    dev = device()
    o, lse = binding.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, tau=tau,
                               out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention(q, k, v, causal, scale)
    tol_o = 2.0 ** -8 + 1e-4 + (0.0 if out_f32 else 2.0 ** -9)
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    note(f"  max|dO| = {eo:.2e} (bound {tol_o:.2e}), max|dLSE| = {el:.2e} (bound 5e-5)")
    assert eo <= tol_o and el <= 5e-5, (eo, el)


def fp8_exact_inputs(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    one, half = 0x38, 0x30
    q8 = torch.zeros((B, H, N, d), dtype=torch.uint8)
    idx = torch.rand((B, H, N, d), generator=g).argsort(dim=-1)[..., :9]  # nine ones per query row
    q8.scatter_(-1, idx, one)
    k8 = torch.where(torch.rand((B, H, N, d), generator=g) < 0.3, one, 0).to(torch.uint8)
    vals = torch.tensor([0x00, half, one, 0x80 | half, 0x80 | one], dtype=torch.uint8)
    v8 = vals[torch.randint(0, 5, (B, H, N, d), generator=g)]
    ldv = binding.fp8_ldv(N)
    vt8 = torch.zeros((B, H, d, ldv), dtype=torch.uint8)
    vt8[..., :N] = v8.transpose(2, 3)
    vt8[..., N:] = 0x7F  # padding holds NaN codes: the kernel must never use it
    return q8, k8, vt8


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_exact_products_leave_only_the_output_rounding(d, causal):
    note(f"fp8 exact: d={d} causal={causal}")
    B, H, N = 1, 2, N_ROWS
    q8, k8, vt8 = fp8_exact_inputs(B, H, N, d, seed=8000 + d + causal)
    scale = float(np.float32(math.log(2.0)))
    assert np.float32(np.float32(scale) * np.float32(1.0) * np.float32(1.0) * np.float32(1.4426950408889634)) == 1.0
    sc = (1.0, 1.0, 1.0)
    dev = device()
    o, lse = binding.attention_fp8(q8.to(dev), k8.to(dev), vt8.to(dev), sc, causal=causal, scale=scale, tau=0.0)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = of.attention_fp8(q8, k8, vt8, sc, causal, scale)
    err = np.abs(o - o_ref)
    bound = 2.0 ** -8 * np.abs(o_ref) + 1e-5
    el = max_err(lse, lse_ref)
    note(f"  max|dO| = {err.max():.2e}, worst |dO| / bound = {(err / bound).max():.3f}, max|dLSE| = {el:.2e}")
    assert np.all(err <= bound) and el <= 1e-5, ((err / bound).max(), el)
