"""Pins for the oracle's several-tokens-per-request (causal) decode.

The reading: the n new tokens of a request are its last n KV tokens, and new
token i sees the KV tokens up to and including its own position. The oracle's
rows are checked against scalar brute force with an explicit causal rule,
against single-token decode of the truncated request (already pinned by the
single-token tests), and a planted off-by-one must be caught.
"""
import math

import numpy as np
import pytest

from oracle import attention
from workloads import custom_workload, explicit_table, host_case

from test_oracle_attention import _scalar


def brute_force_causal(case, sm_scale):
    """Scalar loops: for each new token list the (page, slot) pairs it may see."""
    w = case["workload"]
    q, kv = case["q"], case["kv"]
    indptr, indices, last = case["indptr"], case["indices"], case["last_page_len"]
    qo = case["qo_indptr"]
    Rq, Hq, D = q.shape
    P = kv.shape[2]
    g = Hq // w.num_kv_heads
    out = np.zeros((Rq, Hq, D))
    lse = np.zeros((Rq, Hq))
    for r in range(len(last)):
        pages = [int(p) for p in indices[indptr[r]:indptr[r + 1]]]
        toks = []
        for j, page in enumerate(pages):
            for slot in range(P if j < len(pages) - 1 else int(last[r])):
                toks.append((page, slot))
        n_new = int(qo[r + 1] - qo[r])
        for i in range(n_new):
            row = int(qo[r]) + i
            own_position = len(toks) - n_new + i  # index of this new token in the sequence
            seen = [tok for pos, tok in enumerate(toks) if pos <= own_position]
            for h in range(Hq):
                kvh = h // g
                qv = [_scalar(q[row, h, d], w.q_dtype) for d in range(D)]
                scores, vals = [], []
                for page, slot in seen:
                    ks = vs = 1.0
                    if w.kv_dtype == "e4m3":
                        ks = float(case["k_scale"][page, kvh])
                        vs = float(case["v_scale"][page, kvh])
                    kvec = [_scalar(kv[page, 0, slot, kvh, d], w.kv_dtype) * ks for d in range(D)]
                    vals.append([_scalar(kv[page, 1, slot, kvh, d], w.kv_dtype) * vs
                                 for d in range(D)])
                    scores.append(sm_scale * math.fsum(a * b for a, b in zip(qv, kvec)))
                m = max(scores)
                wts = [math.exp(s - m) for s in scores]
                den = math.fsum(wts)
                for d in range(D):
                    out[row, h, d] = math.fsum(wt * v[d] for wt, v in zip(wts, vals)) / den
                lse[row, h] = m + math.log(den)
    return out, lse


CASES = [
    (1, "f32", "f32", 2, 2, 4, 4, [5, 1, 12], [3, 1, 4]),
    (2, "bf16", "bf16", 4, 2, 8, 4, [9, 16, 3], [1, 5, 3]),
    (3, "e4m3", "bf16", 4, 1, 8, 4, [13, 2, 40], [6, 2, 1]),
]


@pytest.mark.parametrize("seed,kv,qd,hq,hkv,d,p,lens,nq", CASES)
def test_causal_rows_match_brute_force(seed, kv, qd, hq, hkv, d, p, lens, nq):
    w = custom_workload(len(lens), hq, hkv, d, p, kv, qd, lens, pool_pages=sum(lens) // p + 6,
                        qo_lens=nq)
    case = host_case(w, seed, poison=True)
    assert case["qo_indptr"].tolist() == [0] + np.cumsum(nq).tolist()
    out, lse = attention.decode_case(case)
    bo, bl = brute_force_causal(case, w.scale())
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def test_each_row_is_single_token_decode_of_the_truncated_request():
    lens, nq, P = [37, 8, 21], [5, 8, 2], 4
    w = custom_workload(3, 8, 2, 16, P, "bf16", "bf16", lens, pool_pages=40, qo_lens=nq)
    case = host_case(w, 11, poison=True)
    out, lse = attention.decode_case(case)
    qo = case["qo_indptr"]
    for r in range(3):
        pages = case["indices"][case["indptr"][r]:case["indptr"][r + 1]]
        for i in range(nq[r]):
            L = lens[r] - nq[r] + 1 + i
            n = -(-L // P)
            t = explicit_table([pages[:n]], [(L - 1) % P + 1], P, case["kv"].shape[0])
            row = int(qo[r]) + i
            o1, l1 = attention.decode(case["q"][row:row + 1], case["kv"], t["indptr"],
                                      t["indices"], t["last_page_len"], num_kv_heads=2,
                                      q_dtype="bf16", kv_dtype="bf16", sm_scale=w.scale())
            np.testing.assert_array_equal(out[row], o1[0])
            np.testing.assert_array_equal(lse[row], l1[0])


def test_one_token_per_request_equals_plain_decode():
    w = custom_workload(3, 4, 2, 8, 4, "bf16", "bf16", [9, 16, 3], pool_pages=12)
    case = host_case(w, 5, poison=True)
    out0, lse0 = attention.decode_case(case)
    out1, lse1 = attention.decode(case["q"], case["kv"], case["indptr"], case["indices"],
                                  case["last_page_len"], num_kv_heads=2, q_dtype="bf16",
                                  kv_dtype="bf16", sm_scale=w.scale(),
                                  qo_indptr=np.arange(4, dtype=np.int32))
    np.testing.assert_array_equal(out0, out1)
    np.testing.assert_array_equal(lse0, lse1)


def test_last_new_token_sees_the_whole_request():
    """The newest token's row is plain decode over all L tokens."""
    lens, nq = [9, 16, 3], [4, 2, 3]
    w = custom_workload(3, 4, 2, 8, 4, "f32", "f32", lens, pool_pages=12, qo_lens=nq)
    case = host_case(w, 8, poison=True)
    out, _ = attention.decode_case(case)
    last_rows = case["qo_indptr"][1:] - 1
    o1, _ = attention.decode(case["q"][last_rows], case["kv"], case["indptr"], case["indices"],
                             case["last_page_len"], num_kv_heads=2, q_dtype="f32",
                             kv_dtype="f32", sm_scale=w.scale())
    np.testing.assert_array_equal(out[last_rows], o1)


def test_planted_off_by_one_visibility_is_caught(monkeypatch):
    lens, nq = [9, 16, 3], [4, 2, 2]
    w = custom_workload(3, 4, 2, 8, 4, "f32", "f32", lens, pool_pages=12, qo_lens=nq)
    case = host_case(w, 9, poison=True)
    bo, _ = brute_force_causal(case, w.scale())
    monkeypatch.setattr(attention, "visible_tokens", lambda L, n, i: L - n + i)
    out, _ = attention.decode_case(case)
    assert not np.allclose(out, bo, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("bad", [[0, 1, 1, 3], [0, 1, 2, 6], [1, 2, 3, 4]])
def test_invalid_query_layouts_rejected(bad):
    w = custom_workload(3, 4, 2, 8, 4, "f32", "f32", [9, 16, 3], pool_pages=12)
    case = host_case(w, 5, poison=False)
    rows = max(bad[-1], 1)
    q = np.zeros((rows, 4, 8), np.float32)
    with pytest.raises(ValueError):
        attention.decode(q, case["kv"], case["indptr"], case["indices"], case["last_page_len"],
                         num_kv_heads=2, q_dtype="f32", kv_dtype="f32", qo_indptr=bad)
