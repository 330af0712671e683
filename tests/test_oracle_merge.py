"""Pins for the oracle's partial states and merge rule.

The rule itself is the closed form printed in "FlashDecoding + FlashInfer — the
decode-time attention story", §"FlashDecoding — the split-KV trick"; these
tests check that folding partials with it reproduces the unsplit softmax, and
the algebraic properties the rule must have.
"""
import math

import numpy as np
import pytest

from oracle import merge


def _scores_values(n, d, seed, spread=3.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * spread, rng.standard_normal((n, d))


def _direct(s, V):
    w = np.exp(s - s.max())
    return (w @ V) / w.sum(), s.max() + math.log(w.sum())


@pytest.mark.parametrize("seed", range(6))
def test_split_then_merge_equals_unsplit(seed):
    s, V = _scores_values(97, 16, seed)
    ref_o, ref_l = _direct(s, V)
    rng = np.random.default_rng(100 + seed)
    cuts = np.sort(rng.choice(np.arange(1, 97), size=rng.integers(1, 12), replace=False))
    edges = [0, *cuts.tolist(), 97]
    states = [merge.chunk_state(s[a:b], V[a:b]) for a, b in zip(edges[:-1], edges[1:])]
    o, l = merge.finalize(merge.fold(states, 16))
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    assert abs(l - ref_l) < 1e-12


def test_token_by_token_recurrence_equals_softmax():
    """The per-tile recurrence is the merge with one-token states (s_t, 1, v_t)."""
    s, V = _scores_values(40, 8, 3)
    st = merge.identity(8)
    for t in range(40):
        st = merge.merge(st, merge.token_state(s[t], V[t]))
    o, l = merge.finalize(st)
    ref_o, ref_l = _direct(s, V)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    assert abs(l - ref_l) < 1e-12


def test_two_token_closed_form():
    s1, s2 = 0.7, -1.9
    v1, v2 = np.array([1.0, -2.0]), np.array([0.5, 4.0])
    o, l = merge.finalize(merge.merge(merge.token_state(s1, v1), merge.token_state(s2, v2)))
    e1, e2 = math.exp(s1), math.exp(s2)
    np.testing.assert_allclose(o, (e1 * v1 + e2 * v2) / (e1 + e2), rtol=1e-15)
    assert abs(l - math.log(e1 + e2)) < 1e-15


def test_merge_is_commutative_and_associative():
    s, V = _scores_values(30, 4, 8)
    a = merge.chunk_state(s[:7], V[:7])
    b = merge.chunk_state(s[7:19], V[7:19])
    c = merge.chunk_state(s[19:], V[19:])
    ab = merge.merge(a, b)
    ba = merge.merge(b, a)
    assert ab[0] == ba[0]
    np.testing.assert_allclose(ab[1], ba[1], rtol=1e-15)
    np.testing.assert_allclose(ab[2], ba[2], rtol=1e-15)
    left = merge.finalize(merge.merge(ab, c))
    right = merge.finalize(merge.merge(a, merge.merge(b, c)))
    np.testing.assert_allclose(left[0], right[0], rtol=1e-13)


def test_identity_element_and_empty_chunks():
    s, V = _scores_values(5, 3, 1)
    a = merge.chunk_state(s, V)
    e = merge.identity(3)
    for x in (merge.merge(a, e), merge.merge(e, a)):
        assert x[0] == a[0] and x[1] == a[1] and np.array_equal(x[2], a[2])
    both = merge.merge(e, e)
    assert both[0] == -math.inf and both[1] == 0.0 and not np.any(np.isnan(both[2]))
    assert merge.chunk_state(s[:0], V[:0])[0] == -math.inf


def test_merge_is_stable_for_large_score_gaps():
    """exp(m_a - m) never overflows: the larger side's weight is exactly 1."""
    a = merge.token_state(800.0, np.array([1.0]))
    b = merge.token_state(-800.0, np.array([2.0]))
    m, d, o = merge.merge(a, b)
    assert m == 800.0 and d == 1.0 and o[0] == 1.0


def test_split_attend_matches_direct():
    rng = np.random.default_rng(4)
    K, V, q = rng.standard_normal((50, 8)), rng.standard_normal((50, 8)), rng.standard_normal(8)
    o, l = merge.split_attend(q, K, V, 0.3, [(0, 16), (16, 32), (32, 48), (48, 50)])
    ref_o, ref_l = _direct(0.3 * (K @ q), V)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12)
    assert abs(l - ref_l) < 1e-12
