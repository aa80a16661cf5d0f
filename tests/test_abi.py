"""C ABI on the host (CPU only): the library loads, exports what include/attn_fwd.h
declares, and its argument checks return the documented codes without launching."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from exact_attention_22_amd import binding as bnd

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")]

# fake, aligned, non-overlapping device addresses: the checks never dereference them
GB = 1 << 30
Q, K, V, O, L = 1 * GB, 2 * GB, 3 * GB, 4 * GB, 5 * GB


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = bnd.lib()
    names = declared_functions()
    assert set(names) == set(bnd.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert lib.attn_abi_version() == bnd.ABI_VERSION == 10


def check(*args, **kw):
    return bnd.attn_fwd_check(*args, **kw)


def test_valid_arguments_pass():
    assert check(Q, K, V, O, L, 2, 32, 8192, 128, 0, 0.088) == bnd.ATTN_OK
    assert check(Q, K, V, O, L, 1, 1, 1, 64, 1, -3.0) == bnd.ATTN_OK
    assert check(Q, K, V, O, L, 1, 1, 1, 64, 1, 0.0) == bnd.ATTN_OK


def test_empty_is_a_no_op():
    assert check(None, None, None, None, None, 0, 4, 16, 128, 0, 1.0) == bnd.ATTN_OK
    assert check(None, None, None, None, None, 1, 4, 0, 128, 1, 1.0) == bnd.ATTN_OK
    # entry point itself: returns OK without touching the (absent) device
    assert bnd.attn_fwd(None, None, None, None, None, 1, 1, 0, 64, 0, 1.0, None) == bnd.ATTN_OK


@pytest.mark.parametrize("args,code", [
    ((None, K, V, O, L, 1, 1, 8, 64, 0, 1.0), bnd.ATTN_OK + 1),
    ((Q, K, V, O, None, 1, 1, 8, 64, 0, 1.0), 1),
    ((Q, K, V, O, L, -1, 1, 8, 64, 0, 1.0), 2),
    ((Q, K, V, O, L, 1, 1, -8, 64, 0, 1.0), 2),
    ((Q, K, V, O, L, 1 << 20, 1 << 10, 1 << 20, 64, 0, 1.0), 2),
    ((Q, K, V, O, L, 1, 1, (1 << 23), 128, 0, 1.0), 2),
    ((Q, K, V, O, L, 1, 1, 8, 96, 0, 1.0), 3),
    ((Q, K, V, O, L, 1, 1, 8, 256, 0, 1.0), 3),
    ((Q + 8, K, V, O, L, 1, 1, 8, 64, 0, 1.0), 4),
    ((Q, K, V, O + 2, L, 1, 1, 8, 64, 0, 1.0), 4),
    ((Q, K, V, O, L + 2, 1, 1, 8, 64, 0, 1.0), 4),
    ((Q, K, V, O, L, 1, 1, 8, 64, 0, math.inf), 5),
    ((Q, K, V, O, L, 1, 1, 8, 64, 0, math.nan), 5),
    ((Q, K, V, Q, L, 1, 1, 8, 64, 0, 1.0), 6),
    ((Q, K, V, O, V + 64, 1, 1, 8, 64, 0, 1.0), 6),
    ((Q, K, V, O, O + 512, 1, 1, 8, 64, 0, 1.0), 6),
])
def test_error_codes(args, code):
    assert check(*args) == code
    assert bnd.last_error() != ""
    # the entry point reports the same code and launches nothing
    assert bnd.attn_fwd(*args, None) == code


def test_options():
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(tau=0.0)) == bnd.ATTN_OK
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(tau=-1.0)) == 8
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(tau=65.0)) == 8
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(poly_eighths=3)) == 3
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(o_dtype=2)) == 3
    for p8 in (0, 4, 8):
        assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(poly_eighths=p8)) == bnd.ATTN_OK
    small = bnd.make_opts()
    small.struct_size = 8
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, small) == 8
    # fp32 O is twice as large: now overlaps lse placed right after a bf16-sized O
    rows = 1 * 1 * 8
    assert check(Q, K, V, O, O + rows * 64 * 2, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(o_dtype=1)) == 6
    assert check(Q, K, V, O, O + rows * 64 * 2, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(o_dtype=0)) == bnd.ATTN_OK
    # counter buffer: alignment and aliasing
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(rescale_count=L + 2)) == 4
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(rescale_count=L)) == 6
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(rescale_count=6 * GB)) == bnd.ATTN_OK


def test_schedule_option():
    ref = bnd.SCHEDULE_REFERENCE
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(schedule=ref)) == bnd.ATTN_OK
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 1, 0.0, bnd.make_opts(schedule=ref, o_dtype=1)) == bnd.ATTN_OK
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(schedule=2)) == 8
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(schedule=-1)) == 8
    # the reference schedule covers the hardware exponential and scale >= 0 only
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, bnd.make_opts(schedule=ref, poly_eighths=4)) == 3
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, -1.0, bnd.make_opts(schedule=ref)) == 3
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, -1.0, bnd.make_opts()) == bnd.ATTN_OK


def test_options_struct_of_the_previous_abi():
    # a caller built against ABI 8 passes the struct without `schedule` (32 bytes on
    # LP64): the library must not read the field and must use the default
    base = ctypes.sizeof(bnd.AttnFwdOpts) - 8
    assert bnd.AttnFwdOpts.schedule.offset == base == 32
    old = bnd.make_opts(schedule=7)
    old.struct_size = base
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, old) == bnd.ATTN_OK
    old.struct_size = base - 1
    assert check(Q, K, V, O, L, 1, 1, 8, 64, 0, 1.0, old) == 8


def test_tile_shape():
    assert bnd.tile_shape(128)[0] % 32 == 0 and bnd.tile_shape(64)[1] % 32 == 0
    with pytest.raises(bnd.AttnError):
        bnd.tile_shape(96)


def test_status_strings():
    lib = bnd.lib()
    for code in range(9):
        assert lib.attn_status_str(code).decode() not in ("", "unknown status")
    assert lib.attn_status_str(99).decode() == "unknown status"


def test_exp2_polynomial_error_bound():
    """The kernel's software 2^x (the same inline routine, compiled for the host):
    relative error <= 2e-4 against float64 2^x, exact at integers, monotone.
    The pages give no coefficients, only that the polynomial is cubic and reaches
    hardware-level precision (page "FlashAttention 4: faster, more memory-efficient
    attention for LLMs", section "Software exponential on CUDA cores")."""
    lib = bnd.lib()
    f = np.arange(0, 1 << 23, dtype=np.int64).astype(np.float64) / (1 << 23)   # every fp32 in [0,1) ulp-grid
    x = np.concatenate([f.astype(np.float32),
                        np.linspace(-126.0, 64.0, 2_000_001, dtype=np.float32),
                        np.arange(-126, 65, dtype=np.float32)])
    y = np.empty_like(x)
    lib.attn_exp2_poly_host(x.ctypes.data, y.ctypes.data, x.size)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y.astype(np.float64) / ref - 1.0)
    assert rel.max() <= 2e-4, rel.max()
    ints = np.arange(-126, 65, dtype=np.float32)
    yi = np.empty_like(ints)
    lib.attn_exp2_poly_host(ints.ctypes.data, yi.ctypes.data, ints.size)
    assert np.array_equal(yi.astype(np.float64), np.exp2(ints.astype(np.float64)))
    fs = np.sort(x[: 1 << 23])
    ys = np.empty_like(fs)
    lib.attn_exp2_poly_host(fs.ctypes.data, ys.ctypes.data, fs.size)
    assert np.all(np.diff(ys) >= 0)
    # far below (masked keys are -inf): exactly 0, as with the hardware instruction
    lo = np.array([-1e30, -200.0, -151.0, -np.inf], dtype=np.float32)
    ylo = np.empty_like(lo)
    lib.attn_exp2_poly_host(lo.ctypes.data, ylo.ctypes.data, lo.size)
    assert np.all(ylo == 0.0), ylo


def gqa_check(*args, **kw):
    return bnd.attn_fwd_gqa_check(*args, **kw)


def test_gqa_valid_arguments_pass():
    for Hkv in (1, 2, 4, 8, 16, 32):
        assert gqa_check(Q, K, V, O, L, 2, 32, Hkv, 8192, 128, 1, 0.088) == bnd.ATTN_OK
    assert gqa_check(None, None, None, None, None, 1, 0, 0, 16, 64, 0, 1.0) == bnd.ATTN_OK
    assert gqa_check(None, None, None, None, None, 0, 4, 2, 16, 64, 0, 1.0) == bnd.ATTN_OK
    assert bnd.attn_fwd_gqa(None, None, None, None, None, 1, 4, 2, 0, 64, 0, 1.0, None, None) == bnd.ATTN_OK


@pytest.mark.parametrize("H,Hkv", [(32, 0), (32, 3), (32, 64), (6, 4), (4, -1), (0, 1)])
def test_gqa_bad_head_counts(H, Hkv):
    assert gqa_check(Q, K, V, O, L, 1, H, Hkv, 8, 64, 0, 1.0) == 2
    assert "Hkv" in bnd.last_error()
    assert bnd.attn_fwd_gqa(Q, K, V, O, L, 1, H, Hkv, 8, 64, 0, 1.0, None, None) == 2


def test_gqa_alias_uses_key_value_extent():
    """k and v span B*Hkv*N*d elements: an output just past that extent is accepted."""
    B, H, Hkv, N, d = 1, 8, 2, 64, 64
    kv_bytes = B * Hkv * N * d * 2
    assert gqa_check(Q, K, V, K + kv_bytes, L, B, H, Hkv, N, d, 0, 1.0) == bnd.ATTN_OK
    assert gqa_check(Q, K, V, K + kv_bytes - 16, L, B, H, Hkv, N, d, 0, 1.0) == 6
    # the MHA check uses the query extent for k, so the same o overlaps there
    assert check(Q, K, V, K + kv_bytes, L, B, H, N, d, 0, 1.0) == 6


def test_gqa_same_codes_as_mha_when_heads_equal():
    cases = [(Q, K, V, O, L, 1, 4, 8, 96, 0, 1.0), (Q + 8, K, V, O, L, 1, 4, 8, 64, 0, 1.0),
             (Q, K, V, O, L, 1, 4, 8, 64, 0, math.inf), (Q, K, V, Q, L, 1, 4, 8, 64, 0, 1.0)]
    for a in cases:
        g = a[:6] + (a[6],) + a[6:]
        assert check(*a) == gqa_check(*g) != bnd.ATTN_OK


CU = 6 * GB


def varlen_check(*args, **kw):
    return bnd.attn_fwd_varlen_check(*args, **kw)


def test_varlen_valid_arguments_pass():
    # (q, k, v, o, lse, cu, B, H, Hkv, total, max_seqlen, d, causal, scale)
    assert varlen_check(Q, K, V, O, L, CU, 24, 32, 8, 42747, 5753, 128, 1, 0.088) == bnd.ATTN_OK
    assert varlen_check(Q, K, V, O, L, CU, 3, 4, 4, 100, 1000, 64, 0, 1.0) == bnd.ATTN_OK  # max > total
    for empty in [(0, 4, 2, 100, 50), (3, 0, 0, 100, 50), (3, 4, 2, 0, 0), (3, 4, 2, 100, 0)]:
        B, H, Hkv, T, mx = empty
        assert varlen_check(None, None, None, None, None, None, B, H, Hkv, T, mx, 64, 1, 1.0) == bnd.ATTN_OK
        assert bnd.attn_fwd_varlen(None, None, None, None, None, None, B, H, Hkv, T, mx, 64, 1, 1.0,
                                   None, None) == bnd.ATTN_OK


@pytest.mark.parametrize("args,code", [
    ((Q, K, V, O, L, None, 2, 4, 2, 64, 32, 64, 0, 1.0), 1),      # cu_seqlens NULL
    ((Q, K, V, O, L, CU, -1, 4, 2, 64, 32, 64, 0, 1.0), 2),
    ((Q, K, V, O, L, CU, 2, 4, 2, -64, 32, 64, 0, 1.0), 2),
    ((Q, K, V, O, L, CU, 2, 4, 2, 64, -1, 64, 0, 1.0), 2),
    ((Q, K, V, O, L, CU, 2, 4, 3, 64, 32, 64, 0, 1.0), 2),        # Hkv does not divide H
    ((Q, K, V, O, L, CU, 2, 4, 2, 1 << 23, 32, 128, 0, 1.0), 2),  # token axis past 32-bit offsets
    ((Q, K, V, O, L, CU, 2, 4, 2, 64, 32, 96, 0, 1.0), 3),
    ((Q, K, V, O, L, CU + 2, 2, 4, 2, 64, 32, 64, 0, 1.0), 4),
    ((Q, K, V, O, L, CU, 2, 4, 2, 64, 32, 64, 0, math.nan), 5),
    ((Q, K, V, CU - 64, L, CU, 2, 4, 2, 64, 32, 64, 0, 1.0), 6),   # o overlaps cu_seqlens
    ((Q, K, V, O, CU - 4, CU, 2, 4, 2, 64, 32, 64, 0, 1.0), 6),    # lse overlaps cu_seqlens
    ((Q, K, V, O, K + 64, CU, 2, 4, 2, 64, 32, 64, 0, 1.0), 6),
])
def test_varlen_error_codes(args, code):
    assert varlen_check(*args) == code
    assert bnd.last_error() != ""
    assert bnd.attn_fwd_varlen(*args, None, None) == code


def test_varlen_alias_uses_packed_extents():
    """q spans H*total*d elements, k and v Hkv*total*d, lse H*total floats."""
    H, Hkv, T, d = 4, 2, 100, 64
    kv_bytes = Hkv * T * d * 2
    assert varlen_check(Q, K, V, K + kv_bytes, L, CU, 3, H, Hkv, T, 50, d, 0, 1.0) == bnd.ATTN_OK
    assert varlen_check(Q, K, V, K + kv_bytes - 16, L, CU, 3, H, Hkv, T, 50, d, 0, 1.0) == 6
    assert varlen_check(Q, K, V, O, O + H * T * d * 2, CU, 3, H, Hkv, T, 50, d, 0, 1.0) == bnd.ATTN_OK
    assert varlen_check(Q, K, V, O, O + H * T * d * 2 - 4, CU, 3, H, Hkv, T, 50, d, 0, 1.0) == 6


DO, DQ, DK, DV, DL = 7 * GB, 8 * GB, 9 * GB, 10 * GB, 11 * GB


def bwd_check(*args):
    return bnd.attn_bwd_check(*args)


def test_bwd_valid_and_empty():
    # (q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, causal, scale)
    assert bwd_check(Q, K, V, O, L, DO, DQ, DK, DV, DL, 2, 32, 8, 8192, 128, 1, 0.088) == bnd.ATTN_OK
    assert bwd_check(*([None] * 10), 0, 4, 2, 16, 64, 0, 1.0) == bnd.ATTN_OK
    assert bnd.attn_bwd(*([None] * 10), 1, 4, 2, 0, 64, 0, 1.0, None) == bnd.ATTN_OK


def test_bwd_ex_schedule_checked_before_any_launch():
    # an unknown schedule is rejected after the argument checks, before any launch
    # (the pointers are host-side stand-ins; nothing is launched)
    args = [Q, K, V, O, L, DO, DQ, DK, DV, DL, 1, 4, 2, 64, 128, 0, 1.0]
    assert bnd.attn_bwd_ex(*args, 7, None) == 8  # ATTN_ERR_OPTS
    assert "schedule" in bnd.last_error()
    assert bnd.attn_bwd_ex(*args, -1, None) == 8
    # argument errors come first, and an empty problem launches nothing with either schedule
    bad = list(args)
    bad[14] = 96
    assert bnd.attn_bwd_ex(*bad, 1, None) == 3
    empty = [None] * 10 + [1, 4, 2, 0, 128, 0, 1.0]
    for sched in (bnd.SCHEDULE_PIPELINED, bnd.SCHEDULE_REFERENCE):
        assert bnd.attn_bwd_ex(*empty, sched, None) == bnd.ATTN_OK


@pytest.mark.parametrize("patch,code", [
    ({0: None}, 1), ({9: None}, 1), ({12: 3}, 2), ({13: -1}, 2), ({14: 96}, 3), ({16: math.inf}, 5),
    ({6: DQ + 8}, 4), ({9: DL + 2}, 4), ({6: Q}, 6), ({7: DQ + 64}, 6), ({9: V + 4}, 6), ({8: DK}, 6),
])
def test_bwd_error_codes(patch, code):
    args = [Q, K, V, O, L, DO, DQ, DK, DV, DL, 1, 4, 2, 64, 64, 0, 1.0]
    for i, x in patch.items():
        args[i] = x
    assert bwd_check(*args) == code
    assert bnd.last_error() != ""
    assert bnd.attn_bwd(*args, None) == code


def test_splitkv_workspace_size():
    # 8 key tiles of 64 at N = 512; 2 units of 4 tiles: fp32 O and LSE per unit and row
    rows = 1 * 2 * 512
    assert bnd.splitkv_workspace_size(1, 2, 512, 128, 2) == 2 * rows * 128 * 4 + 2 * rows * 4
    assert bnd.splitkv_workspace_size(1, 2, 512, 128, 3) == bnd.splitkv_workspace_size(1, 2, 512, 128, 3)
    # 3 requested -> 3 tiles per unit -> 3 units (8 / 3 rounded up)
    assert bnd.splitkv_workspace_size(1, 2, 512, 64, 3) == 3 * rows * 64 * 4 + 3 * rows * 4
    # more units than key tiles: clamped to 8
    assert bnd.splitkv_workspace_size(1, 2, 512, 64, 100) == 8 * rows * 64 * 4 + 8 * rows * 4
    assert bnd.splitkv_workspace_size(0, 2, 512, 64, 2) == 0
    assert bnd.splitkv_workspace_size(1, 2, 512, 96, 2) == 0
    assert bnd.splitkv_workspace_size(1, 2, 512, 64, -1) == 0


def fp8_check(**kw):
    a = dict(q=Q, k=K, vt=V, o=O, lse=L, B=2, H=32, N=8192, d=128, causal=0, scale=0.088, q_scale=0.01,
             k_scale=0.01, v_scale=0.01, tau=8.0)
    a.update(kw)
    return bnd.attn_fwd_fp8_check(*a.values())


def test_fp8_valid_and_empty():
    assert fp8_check() == bnd.ATTN_OK
    assert fp8_check(N=77, d=64, causal=1, tau=0.0) == bnd.ATTN_OK
    assert fp8_check(q=None, k=None, vt=None, o=None, lse=None, N=0) == bnd.ATTN_OK
    assert bnd.attn_fwd_fp8(None, None, None, None, None, 0, 1, 16, 64, 0, 1.0, 1.0, 1.0, 1.0, 8.0, None) == bnd.ATTN_OK
    for sched in (bnd.SCHEDULE_PIPELINED, bnd.SCHEDULE_REFERENCE):
        assert bnd.attn_fwd_fp8_ex(None, None, None, None, None, 0, 1, 16, 64, 0, 1.0, 1.0, 1.0, 1.0, 8.0, sched,
                                   None) == bnd.ATTN_OK
    # an unknown schedule is an error even where nothing would be launched
    assert bnd.attn_fwd_fp8_ex(None, None, None, None, None, 0, 1, 16, 64, 0, 1.0, 1.0, 1.0, 1.0, 8.0, 2,
                               None) == 8
    # argument errors come first
    assert bnd.attn_fwd_fp8_ex(None, None, None, None, None, 1, 1, 16, 96, 0, 1.0, 1.0, 1.0, 1.0, 8.0, 2,
                               None) == 3


@pytest.mark.parametrize("patch,code", [
    (dict(q=None), 1), (dict(lse=None), 1),
    (dict(B=-1), 2), (dict(N=-3), 2), (dict(B=1 << 20, H=1 << 10, N=1 << 20), 2),
    (dict(B=1, H=1, N=(1 << 24) - 64), 2), (dict(B=1, H=1, N=1 << 25, d=64), 2),  # 32-bit offsets in one head
    (dict(d=96), 3), (dict(tau=8.5), 3), (dict(tau=-1.0), 3), (dict(tau=float("nan")), 3),
    (dict(q=Q + 8), 4), (dict(vt=V + 4), 4), (dict(lse=L + 2), 4),
    (dict(scale=0.0), 5), (dict(scale=-1.0), 5), (dict(q_scale=float("inf")), 5), (dict(v_scale=0.0), 5),
    (dict(scale=1e-30, q_scale=1e-10, k_scale=1e-10), 5),
    (dict(o=Q + 64), 6), (dict(lse=V + 1024), 6), (dict(lse=O + 4096), 6),
])
def test_fp8_error_codes(patch, code):
    assert fp8_check(**patch) == code


def test_fp8_alias_uses_transposed_padded_extent():
    # vt spans B*H*d*ldv bytes with ldv = 8208 for N = 8193: an lse placed inside its padding overlaps
    B, H, N, d = 1, 1, 8193, 64
    ldv = bnd.fp8_ldv(N)
    assert ldv == 8208
    assert fp8_check(B=B, H=H, N=N, d=d, lse=V + d * ldv - 16) == 6
    assert fp8_check(B=B, H=H, N=N, d=d, lse=V + d * ldv) == bnd.ATTN_OK


CU = 12 * GB


def test_bwd_varlen_valid_and_empty():
    # (q, k, v, o, lse, dout, dq, dk, dv, delta, cu, B, H, Hkv, total, max_seqlen, d, causal, scale)
    ok = [Q, K, V, O, L, DO, DQ, DK, DV, DL, CU, 24, 32, 8, 42747, 5753, 128, 1, 0.088]
    assert bnd.attn_bwd_varlen_check(*ok) == bnd.ATTN_OK
    assert bnd.attn_bwd_varlen_check(*([None] * 11), 0, 4, 2, 16, 16, 64, 0, 1.0) == bnd.ATTN_OK
    assert bnd.attn_bwd_varlen_check(*([None] * 11), 3, 4, 2, 16, 0, 64, 0, 1.0) == bnd.ATTN_OK
    assert bnd.attn_bwd_varlen(*([None] * 11), 3, 4, 2, 0, 8, 64, 0, 1.0, None) == bnd.ATTN_OK


@pytest.mark.parametrize("patch,code", [
    ({10: None}, 1), ({0: None}, 1), ({14: -1}, 2), ({15: -1}, 2), ({13: 3}, 2), ({14: 1 << 24}, 2),
    ({16: 80}, 3), ({18: math.nan}, 5), ({10: CU + 2}, 4), ({6: DQ + 8}, 4), ({9: CU}, 6), ({7: DQ + 64}, 6),
])
def test_bwd_varlen_error_codes(patch, code):
    args = [Q, K, V, O, L, DO, DQ, DK, DV, DL, CU, 3, 4, 2, 500, 300, 64, 1, 1.0]
    for i, x in patch.items():
        args[i] = x
    assert bnd.attn_bwd_varlen_check(*args) == code
    assert bnd.last_error() != ""
    assert bnd.attn_bwd_varlen(*args, None) == code
