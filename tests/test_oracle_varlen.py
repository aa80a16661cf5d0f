"""Variable-length (packed) batches in the oracle, pinned (CPU only).

Sequences of different lengths are packed along the token axis (page
"FlashAttention 4: faster, more memory-efficient attention for LLMs", section
"Key points", which lists variable-length batches among the features FA4 lacked).
Layout reading: q [H,total,d], k and v [Hkv,total,d], sequence b owns tokens
cu[b] .. cu[b+1]-1; a query sees only keys of its own sequence.

Pins: a pure-Python brute force that finds each token's sequence by scanning the
bounds and visits every (query, key) pair; the reduction of each sequence to the
dense oracle; isolation between sequences; and planted slips that must fail.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.exact as oa
from exact_attention_22_amd import inputs


def _draw(lengths, H, Hkv, d, seed):
    T = sum(lengths)
    r = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return r.standard_normal((H, T, d)), r.standard_normal((Hkv, T, d)), r.standard_normal((Hkv, T, d)), cu


CASES = [([3, 1, 4], 2, 1, 3), ([5], 2, 2, 2), ([2, 0, 3], 4, 2, 2), ([1, 1, 1, 1], 1, 1, 3), ([6, 2], 3, 3, 2)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[0])) + f"_H{c[1]}_Hkv{c[2]}")
def test_brute_force_varlen(case, causal):
    lengths, H, Hkv, d = case
    q, k, v, cu = _draw(lengths, H, Hkv, d, seed=sum(lengths) + H + causal)
    o1, l1 = oracle.attention_varlen(q, k, v, cu, causal, 0.45)
    o2, l2 = oracle.brute_force_attention_varlen(q, k, v, cu, causal, 0.45)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12


def test_each_sequence_is_the_dense_definition():
    """Sequence b alone, as a dense [1, H, n_b, d] problem, gives the same rows."""
    q, k, v, cu = inputs.draw_varlen([37, 5, 64, 1], 4, 2, 8, seed=51)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cu, causal, 0.3)
        for b in range(4):
            a, e = int(cu[b]), int(cu[b + 1])
            od, ld = oracle.attention_gqa(q[None, :, a:e], k[None, :, a:e], v[None, :, a:e], causal, 0.3)
            assert np.array_equal(od[0], o[:, a:e]) and np.array_equal(ld[0], lse[:, a:e])


def test_sequences_are_isolated():
    """Changing one sequence's queries, keys or values leaves every other sequence bitwise unchanged."""
    q, k, v, cu = inputs.draw_varlen([20, 13, 30], 2, 1, 8, seed=52)
    o, lse = oracle.attention_varlen(q, k, v, cu, True, 0.4)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    a, e = int(cu[1]), int(cu[2])
    q2[:, a:e] += 1.0
    k2[:, a:e] *= -1.0
    v2[:, a:e] += 3.0
    o2, l2 = oracle.attention_varlen(q2, k2, v2, cu, True, 0.4)
    keep = np.r_[0:a, e:int(cu[-1])]
    assert np.array_equal(o[:, keep], o2[:, keep]) and np.array_equal(lse[:, keep], l2[:, keep])
    assert not np.allclose(o[:, a:e], o2[:, a:e])


def test_first_token_of_each_sequence_is_its_value():
    """Causal: a sequence's first token sees only itself, so O = V there and LSE = scale q.k."""
    q, k, v, cu = inputs.draw_varlen([9, 4, 17], 2, 2, 8, seed=53)
    o, lse = oracle.attention_varlen(q, k, v, cu, True, 0.25)
    qf, kf, vf = (t.double().numpy() for t in (q.float(), k.float(), v.float()))
    for b in range(3):
        t = int(cu[b])
        for h in range(2):
            assert np.max(np.abs(o[h, t] - vf[h, t])) <= 1e-15
            assert abs(lse[h, t] - 0.25 * float(qf[h, t] @ kf[h, t])) <= 1e-13


def test_sampled_rows_match_full_varlen():
    q, k, v, cu = inputs.draw_varlen([40, 3, 77, 9], 4, 2, 8, seed=54)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cu, causal, 0.3)
        picks = [(0, [0, 39, 40, 42, 43, 128]), (3, [5]), (2, list(range(129)))]
        for (h, toks), (os_, ls_) in zip(picks, oracle.attention_varlen_rows(q, k, v, cu, causal, 0.3, picks)):
            assert np.max(np.abs(os_ - o[h, toks])) <= 1e-13 and np.max(np.abs(ls_ - lse[h, toks])) <= 1e-13


@pytest.mark.parametrize("cu", [[0, 3, 2, 5], [1, 5], [0, 4], [0, 6]])
def test_bad_bounds_rejected(cu):
    q, k, v, _ = _draw([5], 2, 1, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.attention_varlen(q, k, v, np.array(cu), False, 1.0)


def _mutant(q, k, v, cu, causal, scale, slip):
    """attention_varlen with one plausible slip in the sequence handling."""
    q, k, v = oa._f64(q), oa._f64(k), oa._f64(v)
    H, T, d = q.shape
    Hkv = k.shape[0]
    o = np.empty((H, T, d))
    lse = np.empty((H, T))
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        for h in range(H):
            g = h % Hkv if slip == "head_map_modulo" else h // (H // Hkv)
            if slip == "no_isolation":        # keys of the whole packed batch
                rows = np.arange(a, e)
                o[h, a:e], lse[h, a:e] = oa._rows_of_head(q[h], k[g], v[g], rows, causal, scale)
                continue
            ke = min(T, e + 1) if slip == "bound_off_by_one" else e
            ka = 0 if slip == "keys_from_start" else a
            rows = np.arange(e - a) + (a - ka)
            if e > a:
                o[h, a:e], lse[h, a:e] = oa._rows_of_head(q[h, ka:e], k[g, ka:ke], v[g, ka:ke], rows, causal, scale)
    return o, lse


@pytest.mark.parametrize("slip", ["no_isolation", "bound_off_by_one", "keys_from_start", "head_map_modulo"])
def test_planted_varlen_slip_is_caught(slip):
    caught = False
    for lengths, H, Hkv, d in CASES:
        for causal in (False, True):
            q, k, v, cu = _draw(lengths, H, Hkv, d, seed=77)
            with np.errstate(all="ignore"):
                o1, l1 = _mutant(q, k, v, cu, causal, 0.45, slip)
            o2, l2 = oracle.brute_force_attention_varlen(q, k, v, cu, causal, 0.45)
            caught |= not (np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12)
    assert caught


def test_unmutated_copy_matches_brute_force():
    for lengths, H, Hkv, d in CASES:
        q, k, v, cu = _draw(lengths, H, Hkv, d, seed=78)
        o1, l1 = _mutant(q, k, v, cu, True, 0.45, None)
        o2, l2 = oracle.brute_force_attention_varlen(q, k, v, cu, True, 0.45)
        assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12


def test_varlen_workload_as_stated():
    w = inputs.VARLEN
    L = w.lengths
    assert len(L) == 24 and min(L) >= 64 and max(L) <= 8192 and L == inputs.VARLEN.lengths
    q, k, v, cu = inputs.draw_varlen([5, 7], 4, 2, 8, seed=3)
    assert q.shape == (4, 12, 8) and k.shape == v.shape == (2, 12, 8)
    assert cu.dtype == torch.int32 and cu.tolist() == [0, 5, 12]
