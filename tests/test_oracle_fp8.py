"""FP8 attention in the oracle, pinned (CPU only).

Pins of `oracle.fp8`:
  * the e4m3 decoder against values fixed by the format (bias 7, three mantissa
    bits, subnormals, NaN pattern) and against torch's own float8_e4m3fn
    conversion for all 256 codes;
  * attention of the dequantised codes against a pure-Python brute force that
    decodes through torch (not through the oracle's decoder), with V transposed
    and its padding columns set to NaN codes (never read);
  * the closed form N = 1 (O = v_0, LSE = s_00);
  * the error bound: a CPU simulation of the FP8 kernel's roundings (scores
    perturbed by the dot-product bound, tiles of 64 keys with a lazily updated
    maximum, P rounded to e4m3 by torch, O rounded to bf16) stays inside it,
    and the same bound with its P-rounding term dropped does not.
"""
import math

import numpy as np
import pytest
import torch

import oracle.fp8 as of
from exact_attention_22_amd import inputs


def _torch_decode(c: int) -> float:
    return float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float())


def test_decode_fixed_values():
    # values fixed by the e4m3 field layout (sign | 4 exponent bits, bias 7 | 3 mantissa bits)
    fixed = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x0F: 1.875 * 2.0 ** -6,
             0x77: 240.0, 0x78: 256.0, 0xB8: -1.0, 0x5C: 24.0}
    got = of.e4m3_decode(list(fixed))
    assert np.array_equal(got, np.array(list(fixed.values())))
    assert math.copysign(1.0, float(of.e4m3_decode([0x80])[0])) == -1.0   # negative zero
    assert np.isnan(of.e4m3_decode([0x7F, 0xFF])).all()
    assert np.isfinite(of.e4m3_decode([0x7E, 0x7D, 0x7C, 0x78, 0xF8])).all()   # no infinities


def test_decode_all_codes_match_torch():
    codes = np.arange(256)
    mine = of.e4m3_decode(codes)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_decode_planted_bias_slip_fails():
    c = np.array([0x38, 0x01])
    wrong = (1.0 + (c & 7) / 8.0) * np.exp2(((c >> 3) & 15) - 8.0)
    assert not np.array_equal(wrong, of.e4m3_decode(c))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 5, 4), (2, 1, 7, 3), (1, 1, 17, 2)])
def test_brute_force_fp8(shape, causal):
    B, H, N, d = shape
    g = torch.Generator().manual_seed(sum(shape) + causal)
    q8 = torch.randint(0, 0x70, (B, H, N, d), generator=g).to(torch.uint8) | (torch.randint(0, 2, (B, H, N, d), generator=g).to(torch.uint8) << 7)
    k8 = torch.randint(0, 0x70, (B, H, N, d), generator=g).to(torch.uint8)
    ldv = inputs.fp8_ldv(N)
    vt8 = torch.full((B, H, d, ldv), 0x7F, dtype=torch.uint8)      # padding: NaN codes
    vt8[..., :N] = torch.randint(0, 0x7E, (B, H, d, N), generator=g).to(torch.uint8)
    scales = (0.01, 0.02, 0.5)
    sc = float(np.float32(0.37))
    o1, l1 = of.attention_fp8(q8, k8, vt8, scales, causal, sc)
    o2, l2 = of.brute_force_attention_fp8(q8, k8, vt8, scales, causal, sc, _torch_decode)
    assert np.isfinite(o1).all()
    assert np.max(np.abs(o1 - o2)) <= 1e-9 * max(1.0, np.abs(o2).max())
    assert np.max(np.abs(l1 - l2)) <= 1e-9 * max(1.0, np.abs(l2).max())


def test_brute_force_catches_untransposed_v():
    """Reading vt as if it were [N, d] must disagree with the brute force."""
    B, H, N, d = 1, 1, 4, 4
    q8, k8, vt8, sc = inputs.draw_fp8(B, H, N, d, seed=3)
    vt8 = vt8[..., :N].contiguous()
    wrong = vt8.transpose(-1, -2).contiguous()
    o1, _ = of.attention_fp8(q8, k8, wrong, sc, False, 0.5)
    o2, _ = of.brute_force_attention_fp8(q8, k8, vt8, sc, False, 0.5, _torch_decode)
    assert np.max(np.abs(o1 - o2)) > 1e-3


def test_single_key_closed_form():
    q8, k8, vt8, sc = inputs.draw_fp8(2, 3, 1, 64, seed=11)
    o, lse = of.attention_fp8(q8, k8, vt8, sc, False, 0.125)
    v0 = of.e4m3_decode(vt8[..., 0].numpy()) * np.float32(sc[2])
    s = 0.125 * np.einsum("bhd,bhd->bh", of.e4m3_decode(q8[:, :, 0].numpy()) * np.float32(sc[0]),
                          of.e4m3_decode(k8[:, :, 0].numpy()) * np.float32(sc[1]))
    assert np.max(np.abs(o[:, :, 0] - v0)) <= 1e-15
    assert np.max(np.abs(lse[:, :, 0] - s)) <= 1e-12


# Largest e4m3 dot-product error the gfx950 matrix core showed, relative to
# sum_k |a_k b_k|, over 4 194 304 dot products of 64 codes drawn uniformly over
# every finite e4m3 value (profiles/fp8_mfma_dot_error.md, written by
# exact_attention_22_amd/micro/fp8_dot_error.hip). A device measurement, kept apart
# from the oracle's bound EPS_DOT so that the two check each other.
MEASURED_DOT_REL = 3.211e-4  # 2^-11.60
EPS_DOT_MAX_FACTOR = 8.0     # the bound may exceed the measurement by at most this factor


def test_dot_bound_covers_the_measurement_and_stays_near_it():
    """EPS_DOT must cover what the device did, and must not be so loose that the FP8
    parity bound loses its teeth (a bound 10x too wide fails here)."""
    assert of.EPS_DOT >= MEASURED_DOT_REL
    assert of.EPS_DOT <= EPS_DOT_MAX_FACTOR * MEASURED_DOT_REL


def _simulate_fp8_kernel(q, k, v, causal, scale, eps_dot, tau=8.0, bc=64, seed=0):
    """CPU model of the FP8 kernel's roundings for one head (float64 otherwise): every score
    perturbed by +-E (E = eps_dot * max_j sum_k |scale q_k k_k|), 64-key tiles with a maximum
    that moves only when a tile exceeds it by more than tau (log2 units), P rounded to e4m3
    (torch, round to nearest even), row sum from the unrounded P, O rounded to bf16."""
    r = np.random.default_rng(seed)
    N = q.shape[0]
    s = scale * (q @ k.T)
    t = abs(scale) * (np.abs(q) @ np.abs(k.T))
    E = eps_dot * t.max(axis=1, keepdims=True)
    s = s + E * r.choice([-1.0, 1.0], size=s.shape)
    if causal:
        s = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s, -np.inf)
    x = s / math.log(2.0)
    O = np.zeros_like(q[:, :1] * 0 + v[:1] * 0)
    for i in range(N):
        m = -np.inf
        l = 0.0
        acc = np.zeros(v.shape[1])
        for j0 in range(0, N, bc):
            xt = x[i, j0:j0 + bc]
            mt = xt.max()
            if mt > m + tau:
                alpha = 0.0 if m == -np.inf else 2.0 ** (m - mt)
                l *= alpha
                acc *= alpha
                m = mt
            p = np.exp2(xt - m)
            l += p.sum()
            pq = torch.from_numpy(p).float().to(torch.float8_e4m3fn).double().numpy()
            acc += pq @ v[j0:j0 + bc]
        O[i] = acc / l
    return torch.from_numpy(O).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("causal,drift", [(False, False), (True, False), (True, True)])
def test_error_bound_contains_simulated_roundings(causal, drift):
    q8, k8, vt8, sc = inputs.draw_fp8(1, 2, 160, 64, seed=31 + causal + 2 * drift, drift=drift)
    scale = float(np.float32(1 / 8))
    o_ref, _ = of.attention_fp8(q8, k8, vt8, sc, causal, scale)
    bo, bl = of.fp8_error_bound(q8, k8, vt8, sc, causal, scale)
    q, k, v = of.dequantize(q8, k8, vt8, 160, sc)
    worst = 0.0
    for h in range(2):
        # the simulated kernel perturbs every score by the measured device error, so a
        # bound (EPS_DOT) below the device's behaviour would be violated here
        osim = _simulate_fp8_kernel(q[0, h], k[0, h], v[0, h], causal, scale, MEASURED_DOT_REL, seed=h)
        err = np.abs(osim - o_ref[0, h]).max(axis=1)
        assert np.all(err <= bo[0, h]), float((err / bo[0, h]).max())
        worst = max(worst, float((err / bo[0, h]).max()))
    assert worst > 0.02          # the bound is not vacuous by orders of magnitude
    assert np.all(bl > 0) and np.all(bl < 2e-2)


def test_error_bound_without_p_term_fails():
    """Planted slip: a bound that forgets the e4m3 rounding of P is violated by the simulation."""
    q8, k8, vt8, sc = inputs.draw_fp8(1, 1, 160, 64, seed=41)
    scale = float(np.float32(1 / 8))
    o_ref, _ = of.attention_fp8(q8, k8, vt8, sc, False, 0.125)
    q, k, v = of.dequantize(q8, k8, vt8, 160, sc)
    osim = _simulate_fp8_kernel(q[0, 0], k[0, 0], v[0, 0], False, scale, MEASURED_DOT_REL)
    err = np.abs(osim - o_ref[0, 0]).max(axis=1)
    saved = of.P_REL, of.P_ABS
    try:
        of.P_REL, of.P_ABS = 0.0, 0.0
        bo, _ = of.fp8_error_bound(q8, k8, vt8, sc, False, scale)
    finally:
        of.P_REL, of.P_ABS = saved
    assert np.any(err > bo[0, 0])


def test_rows_match_full():
    q8, k8, vt8, sc = inputs.draw_fp8(2, 2, 70, 64, seed=5)
    o, l = of.attention_fp8(q8, k8, vt8, sc, True, 0.125)
    bo, bl = of.fp8_error_bound(q8, k8, vt8, sc, True, 0.125)
    picks = [(1, 0, [0, 33, 69]), (0, 1, [5])]
    rows = of.attention_fp8_rows(q8, k8, vt8, sc, True, 0.125, picks)
    brows = of.fp8_error_bound_rows(q8, k8, vt8, sc, True, 0.125, picks)
    for (b, h, r), (orow, lrow), (bor, blr) in zip(picks, rows, brows):
        assert np.allclose(orow, o[b, h, r], rtol=1e-12, atol=1e-14) and np.allclose(lrow, l[b, h, r], rtol=1e-12)
        assert np.allclose(bor, bo[b, h, r], rtol=1e-12) and np.allclose(blr, bl[b, h, r], rtol=1e-12)
