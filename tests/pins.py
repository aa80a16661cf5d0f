"""Checks that pin an attention implementation to facts fixed by the mathematics.

Each check takes `fn(q, k, v, causal, scale) -> (O, LSE)` working in float64 on
[B,H,N,d] arrays and raises AssertionError when the implementation is wrong.
They are applied to the oracle (which must pass every one) and to planted
mistakes in copies of it (each of which must fail at least one), so that a
plausible slip anywhere in the oracle is caught by something other than the
oracle itself.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _eval(expr: str) -> float:
    ns = {"exp": math.exp, "log": math.log, "tanh": math.tanh, "e": math.e}
    return float(eval(expr, {"__builtins__": {}}, ns))  # fixture expressions only


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def check_golden(fn):
    """Hand-worked closed-form cases (tests/golden/closed_forms.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(c[x], dtype=np.float64) for x in "qkv")
        for mode, causal in (("noncausal", False), ("causal", True)):
            exp_o = np.vectorize(_eval)(np.array(c[mode]["O"], dtype=object)).astype(np.float64)
            exp_l = np.vectorize(_eval)(np.array(c[mode]["LSE"], dtype=object)).astype(np.float64)
            o, lse = fn(q, k, v, causal, c["scale"])
            _close(o, exp_o, what=f"{c['name']} {mode} O")
            _close(lse, exp_l, what=f"{c['name']} {mode} LSE")


def check_single_key(fn):
    """N=1: the only key gets weight 1, so O = V[0] and LSE = scale * q0.k0."""
    r = _rng(1)
    q, k, v = (r.standard_normal((2, 3, 1, 8)) for _ in range(3))
    for causal in (False, True):
        o, lse = fn(q, k, v, causal, 0.3)
        _close(o, v, what="N=1 O")
        _close(lse, 0.3 * np.einsum("bhid,bhid->bhi", q, k), what="N=1 LSE")


def check_zero_scale(fn):
    """scale = 0: uniform weights over the visible keys; LSE = ln |J(i)|."""
    r = _rng(2)
    B, H, N, d = 1, 2, 9, 4
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    o, lse = fn(q, k, v, False, 0.0)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), what="scale0 O")
    _close(lse, np.full((B, H, N), math.log(N)), what="scale0 LSE")
    o, lse = fn(q, k, v, True, 0.0)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    _close(o, prefix_mean, what="scale0 causal O")
    _close(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N)), what="scale0 causal LSE")


def check_constant_values(fn):
    """All value rows equal: any convex combination returns that row."""
    r = _rng(3)
    q, k = r.standard_normal((2, 2, 11, 8)), r.standard_normal((2, 2, 11, 8))
    row = r.standard_normal(8)
    v = np.broadcast_to(row, q.shape).copy()
    for causal in (False, True):
        o, _ = fn(q, k, v, causal, 0.4)
        _close(o, v, what="constant V")


def check_causal_first_row(fn):
    """Causal row 0 sees key 0 only: O0 = V0, LSE0 = scale * q0.k0."""
    r = _rng(4)
    q, k, v = (r.standard_normal((1, 3, 7, 8)) for _ in range(3))
    o, lse = fn(q, k, v, True, 0.7)
    _close(o[:, :, 0], v[:, :, 0], what="causal row0 O")
    _close(lse[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), what="causal row0 LSE")


def check_dominant_key(fn):
    """One key with a logit gap of at least 60 nats: O equals that key's value to e^-60."""
    B, H, N, d = 1, 1, 6, 3
    q = np.zeros((B, H, N, d)); q[..., 0] = 1.0
    k = np.zeros((B, H, N, d)); k[0, 0, 4, 0] = 60.0
    r = _rng(5)
    v = r.standard_normal((B, H, N, d))
    o, lse = fn(q, k, v, False, 1.0)
    _close(o, np.broadcast_to(v[:, :, 4:5], o.shape), what="dominant O")
    _close(lse, np.full((B, H, N), 60.0 + math.log1p(5 * math.exp(-60))), what="dominant LSE")


def check_key_value_permutation(fn):
    """Non-causal: permuting key and value rows together leaves O and LSE unchanged."""
    r = _rng(6)
    q, k, v = (r.standard_normal((1, 2, 10, 4)) for _ in range(3))
    perm = r.permutation(10)
    o1, l1 = fn(q, k, v, False, 0.5)
    o2, l2 = fn(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    _close(o1, o2, what="kv permutation O")
    _close(l1, l2, what="kv permutation LSE")
    # permuting the queries permutes the outputs
    o3, l3 = fn(q[:, :, perm], k, v, False, 0.5)
    _close(o3, o1[:, :, perm], what="q permutation O")
    _close(l3, l1[:, :, perm], what="q permutation LSE")


def check_key_shift(fn):
    """Adding w to every key adds scale*q_i.w to every score of row i: O is unchanged, LSE_i += scale*q_i.w."""
    r = _rng(7)
    q, k, v = (r.standard_normal((1, 2, 9, 4)) for _ in range(3))
    w = r.standard_normal(4)
    for causal in (False, True):
        o1, l1 = fn(q, k, v, causal, 0.6)
        o2, l2 = fn(q, k + w, v, causal, 0.6)
        _close(o2, o1, tol=1e-11, what="key shift O")
        _close(l2, l1 + 0.6 * (q @ w), tol=1e-11, what="key shift LSE")


def check_causal_prefix(fn):
    """Causal rows < n do not depend on keys, values or queries at positions >= n."""
    r = _rng(8)
    q, k, v = (r.standard_normal((1, 2, 12, 4)) for _ in range(3))
    o1, l1 = fn(q, k, v, True, 0.5)
    n = 5
    o2, l2 = fn(q[:, :, :n], k[:, :, :n], v[:, :, :n], True, 0.5)
    _close(o1[:, :, :n], o2, what="causal prefix O")
    _close(l1[:, :, :n], l2, what="causal prefix LSE")


def check_heads_independent(fn):
    """Each (b, h) equals a separate single-head run on that head's slices."""
    r = _rng(9)
    q, k, v = (r.standard_normal((2, 3, 6, 4)) for _ in range(3))
    for causal in (False, True):
        o, lse = fn(q, k, v, causal, 0.8)
        for b in range(2):
            for h in range(3):
                sl = (slice(b, b + 1), slice(h, h + 1))
                o1, l1 = fn(q[sl], k[sl], v[sl], causal, 0.8)
                _close(o[sl], o1, what="head independence O")
                _close(lse[sl], l1, what="head independence LSE")


def check_probability_rows(fn):
    """O with V = identity rows recovers the softmax: each row sums to 1 and is non-negative."""
    r = _rng(10)
    N = 8
    q, k = r.standard_normal((1, 1, N, N)), r.standard_normal((1, 1, N, N))
    v = np.eye(N)[None, None]
    for causal in (False, True):
        p, _ = fn(q, k, v, causal, 0.9)
        _close(p.sum(axis=-1), np.ones((1, 1, N)), what="P rows sum")
        assert p.min() >= 0.0
        if causal:
            assert np.all(p[0, 0][np.triu_indices(N, 1)] == 0.0), "causal P above diagonal"


ALL_CHECKS = [
    check_golden, check_single_key, check_zero_scale, check_constant_values,
    check_causal_first_row, check_dominant_key, check_key_value_permutation,
    check_key_shift, check_causal_prefix, check_heads_independent, check_probability_rows,
]
