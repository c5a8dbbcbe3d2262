"""CPU pins of the oracle's partial attention over a key range and its merge.

``partial`` and ``merge`` are checked against things other than themselves:
the full reference (itself pinned in test_oracle_attention.py), the tail rows
of a longer problem (which fixes the meaning of the query position), a scalar
brute force for a non-square causal case, and the identities of the merge.
"""
import math

import numpy as np
import pytest

from oracle import attention as A

RNG = np.random.default_rng(2024)


def _qkv(nq, nk, d, b=1, h=2):
    q = RNG.standard_normal((b, h, nq, d))
    k = RNG.standard_normal((b, h, nk, d))
    v = RNG.standard_normal((b, h, nk, d))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 64), (0, 10, 64), (0, 0, 33, 33, 64), (0, 1, 2, 63, 64), (0, 31, 32, 40, 64)])
def test_merged_partials_equal_the_full_reference(causal, cuts):
    q, k, v = _qkv(64, 64, 8)
    o, l = A.reference(q, k, v, causal, 0.4)
    parts = [A.partial(q, k, v, causal, 0.4, 0, a, b) for a, b in zip(cuts, cuts[1:])]
    om, lm = A.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.abs(om - o).max() < 1e-12 and np.abs(lm - l).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_query_position_means_the_tail_of_a_longer_problem(causal):
    """Queries at positions N-Nq .. N-1 against all N keys = the last Nq rows of the square problem."""
    n, nq = 90, 7
    q, k, v = _qkv(n, n, 8)
    o, l = A.reference(q, k, v, causal, 0.25)
    op, lp = A.partial(q[:, :, n - nq:], k, v, causal, 0.25, n - nq, 0, n)
    assert np.abs(op - o[:, :, n - nq:]).max() < 1e-12 and np.abs(lp - l[:, :, n - nq:]).max() < 1e-12


def test_partial_matches_bruteforce_non_square_causal():
    nq, nk, d, pos0, kb, ke, scale = 4, 9, 3, 3, 2, 8, 0.7
    q, k, v = _qkv(nq, nk, d, b=1, h=1)
    op, lp = A.partial(q, k, v, True, scale, pos0, kb, ke)
    for i in range(nq):
        vis = [j for j in range(kb, ke) if j <= pos0 + i]
        if not vis:
            assert lp[0, 0, i] == -np.inf and not op[0, 0, i].any()
            continue
        s = {j: scale * math.fsum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in vis}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in vis}
        z = math.fsum(w.values())
        for c in range(d):
            assert abs(op[0, 0, i, c] - math.fsum(w[j] * v[0, 0, j, c] for j in vis) / z) < 1e-13
        assert abs(lp[0, 0, i] - (m + math.log(z))) < 1e-13


def test_empty_ranges_and_rows():
    q, k, v = _qkv(16, 40, 8)
    o, l = A.partial(q, k, v, False, 0.3, 0, 12, 12)  # empty range
    assert not o.any() and np.all(l == -np.inf)
    o, l = A.partial(q, k, v, True, 0.3, 0, 20, 40)  # causal: query i sees keys <= i < 20
    assert not o.any() and np.all(l == -np.inf)
    o, l = A.partial(q, k, v, True, 0.3, 10, 20, 40)  # rows 0..9 see nothing, rows 10.. see 20..10+i
    assert not o[:, :, :10].any() and np.all(l[:, :, :10] == -np.inf) and np.all(np.isfinite(l[:, :, 10:]))


def test_merge_identities():
    q, k, v = _qkv(20, 50, 8)
    o, l = A.partial(q, k, v, True, 0.3, 30, 0, 50)
    om, lm = A.merge(o[None], l[None])  # one part: unchanged
    assert np.abs(om - o).max() < 1e-15 and np.abs(lm - l).max() < 1e-15
    e_o, e_l = A.partial(q, k, v, True, 0.3, 30, 50, 50)  # adding an empty part changes nothing
    om, lm = A.merge(np.stack([e_o, o]), np.stack([e_l, l]))
    assert np.abs(om - o).max() < 1e-15 and np.abs(lm - l).max() < 1e-15
    # order of the parts does not matter
    a, b = A.partial(q, k, v, True, 0.3, 30, 0, 17), A.partial(q, k, v, True, 0.3, 30, 17, 50)
    o1, l1 = A.merge(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
    o2, l2 = A.merge(np.stack([b[0], a[0]]), np.stack([b[1], a[1]]))
    assert np.abs(o1 - o2).max() < 1e-14 and np.abs(l1 - l2).max() < 1e-14
