"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is the oracle's per-head row routine with one plausible slip (a
dropped term, a wrong sign or index, a transposed operand). It is planted in
the oracle module with monkeypatch, and at least one pin in tests/pins.py must
then fail. This shows the pins constrain every part of the oracle.
"""
import numpy as np
import pytest

import oracle.exact as oa
from tests import pins


def _base(qh, kh, vh, rows, causal, scale, slip):
    rows = np.asarray(rows)
    if slip == "qk_swapped":
        s = scale * (kh[rows] @ qh.T)
    elif slip == "no_scale":
        s = qh[rows] @ kh.T
    elif slip == "scale_twice":
        s = scale * scale * (qh[rows] @ kh.T)
    else:
        s = scale * (qh[rows] @ kh.T)
    if causal:
        keys = np.arange(kh.shape[0])[None, :]
        if slip == "mask_strict":
            vis = keys < rows[:, None]
        elif slip == "mask_transposed":
            vis = keys >= rows[:, None]
        elif slip == "mask_off_by_one":
            vis = keys <= rows[:, None] + 1
        else:
            vis = keys <= rows[:, None]
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m) if slip != "max_sign" else np.exp(s + m)
    l = e.sum(axis=1, keepdims=True)
    if slip == "values_are_keys":
        o = (e @ kh) / l
    elif slip == "no_normalise":
        o = e @ vh
    elif slip == "value_feature_reversed":
        o = (e @ vh[:, ::-1]) / l
    else:
        o = (e @ vh) / l
    if slip == "lse_no_max":
        lse = np.log(l[:, 0])
    elif slip == "lse_log2":
        lse = m[:, 0] + np.log2(l[:, 0])
    elif slip == "lse_max_sign":
        lse = -m[:, 0] + np.log(l[:, 0])
    else:
        lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


SLIPS = ["qk_swapped", "no_scale", "scale_twice", "mask_strict", "mask_transposed",
         "mask_off_by_one", "max_sign", "values_are_keys", "no_normalise",
         "value_feature_reversed", "lse_no_max", "lse_log2", "lse_max_sign"]


def _run_pins():
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(lambda q, k, v, c, s: oa.attention(q, k, v, c, s))
        except (AssertionError, ValueError, FloatingPointError) as exc:
            failures.append((check.__name__, str(exc)[:80]))
    return failures


def test_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(oa, "_rows_of_head", lambda *a: _base(*a, slip=None))
    assert _run_pins() == []


@pytest.mark.parametrize("slip", SLIPS)
def test_planted_mistake_is_caught(monkeypatch, slip):
    monkeypatch.setattr(oa, "_rows_of_head", lambda *a: _base(*a, slip=slip))
    assert _run_pins(), f"no pin caught the planted mistake {slip!r}"
