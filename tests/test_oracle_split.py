"""The split-key merge against the definition (CPU only).

Split keys compute, for each key range s, the attention of a query row over
that range alone (O_s, LSE_s) and merge them with LSE = log sum_s exp(LSE_s),
O = sum_s exp(LSE_s - LSE) O_s. Exact attention over all keys is the plain
definition (the oracle); this pins that the merge, as the HIP path performs it,
reproduces it, including ranges a causal row does not reach (left out).
"""
import numpy as np
import pytest

import oracle


def partial(qh, kh, vh, rows, keys, causal, scale):
    """Attention of `rows` over the key index set `keys` only (None where a row sees none)."""
    with np.errstate(all="ignore"):
        s = scale * (qh[rows] @ kh[keys].T)
        vis = np.ones_like(s, dtype=bool) if not causal else keys[None, :] <= rows[:, None]
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        seen = np.isfinite(m[:, 0])
        e = np.exp(np.where(seen[:, None], s - m, -np.inf))
        l = e.sum(axis=1, keepdims=True)
        return (e @ vh[keys]) / l, m[:, 0] + np.log(l[:, 0]), seen


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [[0, 64, 128, 200], [0, 1, 200], [0, 199, 200], [0, 50, 100, 150, 200]])
def test_merge_reproduces_definition(cuts, causal):
    r = np.random.default_rng(len(cuts) + causal)
    q, k, v = (r.standard_normal((1, 2, 200, 16)) for _ in range(3))
    o_ref, lse_ref = oracle.attention(q, k, v, causal, 0.3)
    rows = np.arange(200)
    for h in range(2):
        parts = [partial(q[0, h], k[0, h], v[0, h], rows, np.arange(a, b), causal, 0.3)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        with np.errstate(all="ignore"):
            lse_s = np.stack([np.where(seen, l, -np.inf) for _, l, seen in parts])
            m = lse_s.max(axis=0)
            lse = m + np.log(np.exp(lse_s - m).sum(axis=0))
            o = sum(np.where(seen[:, None], np.exp(np.where(seen, l, -np.inf) - lse)[:, None] * np.nan_to_num(ob),
                             0.0) for ob, l, seen in parts)
        assert np.max(np.abs(o - o_ref[0, h])) <= 1e-12 and np.max(np.abs(lse - lse_ref[0, h])) <= 1e-12
