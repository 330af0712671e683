"""Pins for cascade attention in the oracle: a shared prefix attended once by
all of its requests' queries (non-causal rows), each request's own suffix
attended separately, and the two normalised results merged.

The pin is the definition itself: the merged result must equal plain decode of
each request over its prefix pages followed by its suffix pages, and merging
with a result over no tokens must change nothing.
"""
import math

import numpy as np
import pytest

from oracle import attention, merge
from workloads import custom_workload, explicit_table, host_case


def _split_tables(P, prefix_pages, suffix_lists, suffix_last, num_pages):
    """Page tables of the full requests, of the suffixes, and of the prefix."""
    full = explicit_table([prefix_pages + s for s in suffix_lists], suffix_last, P, num_pages)
    suffix = explicit_table(suffix_lists, suffix_last, P, num_pages)
    prefix = explicit_table([prefix_pages], [P], P, num_pages)
    return full, suffix, prefix


@pytest.mark.parametrize("kv,qd", [("f32", "f32"), ("bf16", "bf16"), ("e4m3", "bf16")])
def test_cascade_equals_decode_over_prefix_plus_suffix(kv, qd):
    P, B = 4, 5
    rng = np.random.default_rng(3)
    pool = 40
    perm = rng.permutation(pool).tolist()
    prefix_pages = perm[:6]
    suffix_lists = [perm[6 + 3 * r: 6 + 3 * r + 1 + r % 3] for r in range(B)]
    suffix_last = [1 + r % P for r in range(B)]
    full, suffix, prefix = _split_tables(P, prefix_pages, suffix_lists, suffix_last, pool)
    w = custom_workload(B, 8, 2, 16, P, kv, qd, full["kv_lens"].tolist(), pool_pages=pool)
    case = host_case(w, 11, poison=False, table=full)
    kw = dict(num_kv_heads=2, q_dtype=qd, kv_dtype=kv, sm_scale=w.scale(),
              k_scale=case["k_scale"], v_scale=case["v_scale"])
    ref, ref_lse = attention.decode(case["q"], case["kv"], full["indptr"], full["indices"],
                                    full["last_page_len"], **kw)
    # level 0: every request's query attends to the one shared prefix, non-causally
    o0, l0 = attention.decode(case["q"], case["kv"], prefix["indptr"], prefix["indices"],
                              prefix["last_page_len"], qo_indptr=[0, B], causal=False, **kw)
    # level 1: each request's own suffix
    o1, l1 = attention.decode(case["q"], case["kv"], suffix["indptr"], suffix["indices"],
                              suffix["last_page_len"], **kw)
    out, lse = merge.merge_normalized(o0, l0, o1, l1)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_non_causal_rows_each_equal_one_token_decode():
    """Non-causal rows of one request are independent one-token decodes."""
    w = custom_workload(2, 4, 1, 8, 4, "f32", "f32", [9, 6], pool_pages=8)
    case = host_case(w, 2, poison=True)
    q = np.random.default_rng(0).standard_normal((7, 4, 8)).astype(np.float32)
    out, lse = attention.decode(q, case["kv"], case["indptr"], case["indices"],
                                case["last_page_len"], num_kv_heads=1, q_dtype="f32",
                                kv_dtype="f32", qo_indptr=[0, 3, 7], causal=False)
    for row, r in enumerate([0, 0, 0, 1, 1, 1, 1]):
        t = explicit_table([case["indices"][case["indptr"][r]:case["indptr"][r + 1]]],
                           [case["last_page_len"][r]], 4, case["kv"].shape[0])
        o1, l1 = attention.decode(q[row:row + 1], case["kv"], t["indptr"], t["indices"],
                                  t["last_page_len"], num_kv_heads=1, q_dtype="f32",
                                  kv_dtype="f32")
        np.testing.assert_array_equal(out[row], o1[0])
        np.testing.assert_array_equal(lse[row], l1[0])


def test_merge_normalized_closed_forms():
    rng = np.random.default_rng(1)
    va, vb = rng.standard_normal((3, 5)), rng.standard_normal((3, 5))
    la, lb = rng.standard_normal(3), rng.standard_normal(3)
    out, lse = merge.merge_normalized(va, la, vb, lb)
    wa, wb = np.exp(la), np.exp(lb)
    np.testing.assert_allclose(out, (va * wa[:, None] + vb * wb[:, None]) / (wa + wb)[:, None],
                               rtol=1e-13)
    np.testing.assert_allclose(lse, np.logaddexp(la, lb), rtol=1e-13)
    # an empty side (lse = -inf) is the identity
    out, lse = merge.merge_normalized(va, la, np.zeros_like(vb), np.full(3, -math.inf))
    np.testing.assert_array_equal(out, va)
    np.testing.assert_array_equal(lse, la)
    # equal lse: the plain average, lse + ln 2
    out, lse = merge.merge_normalized(va, la, vb, la)
    np.testing.assert_allclose(out, (va + vb) / 2, rtol=1e-13)
    np.testing.assert_allclose(lse, la + math.log(2), rtol=1e-13)
