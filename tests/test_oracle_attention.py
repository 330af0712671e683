"""Pins for the oracle's decode-attention definition.

Each test checks ``oracle.attention`` against something other than itself:
pure-Python brute force, torch's float64 attention on dense K/V, closed forms,
invariants, and the worked page-table example of "FlashDecoding + FlashInfer —
the decode-time attention story", §"Paged attention (vLLM)".
"""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import attention
from workloads import custom_workload, explicit_table, host_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ brute force

def _scalar(x, dtype):
    """One stored value -> Python float, without the oracle's helpers."""
    if dtype in ("f32", "f16"):
        return float(x)
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]
    if dtype == "e4m3":
        t = torch.tensor([int(x)], dtype=torch.uint8).view(torch.float8_e4m3fn)
        return float(t.to(torch.float64)[0])
    raise ValueError(dtype)


def brute_force(case, sm_scale):
    """Scalar loops and math.fsum: walk each page list slot by slot."""
    w = case["workload"]
    q, kv = case["q"], case["kv"]
    indptr, indices, last = case["indptr"], case["indices"], case["last_page_len"]
    B, Hq, D = q.shape
    P = kv.shape[2]
    g = Hq // w.num_kv_heads
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    lse = [[0.0] * Hq for _ in range(B)]
    for r in range(B):
        pages = [int(p) for p in indices[indptr[r]:indptr[r + 1]]]
        toks = []
        for i, page in enumerate(pages):
            used = P if i < len(pages) - 1 else int(last[r])
            for slot in range(used):
                toks.append((page, slot))
        for h in range(Hq):
            kvh = h // g
            qv = [_scalar(q[r, h, d], w.q_dtype) for d in range(D)]
            scores, vals = [], []
            for page, slot in toks:
                ks = vs = 1.0
                if w.kv_dtype == "e4m3" and case["k_scale"].ndim == 3:  # per token
                    ks = float(case["k_scale"][page, kvh, slot])
                    vs = float(case["v_scale"][page, kvh, slot])
                elif w.kv_dtype == "e4m3":
                    ks = float(case["k_scale"][page, kvh])
                    vs = float(case["v_scale"][page, kvh])
                kvec = [_scalar(kv[page, 0, slot, kvh, d], w.kv_dtype) * ks for d in range(D)]
                vvec = [_scalar(kv[page, 1, slot, kvh, d], w.kv_dtype) * vs for d in range(D)]
                scores.append(sm_scale * math.fsum(a * b for a, b in zip(qv, kvec)))
                vals.append(vvec)
            m = max(scores)
            wts = [math.exp(s - m) for s in scores]
            den = math.fsum(wts)
            for d in range(D):
                out[r][h][d] = math.fsum(wt * v[d] for wt, v in zip(wts, vals)) / den
            lse[r][h] = m + math.log(den)
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed,kv_dtype,q_dtype,hq,hkv,d,p,lens", [
    (1, "f32", "f32", 2, 2, 4, 4, [5, 1, 12]),
    (2, "bf16", "bf16", 4, 2, 8, 4, [9, 16, 3]),
    (3, "bf16", "f32", 6, 2, 4, 2, [7, 1]),
    (4, "e4m3", "bf16", 4, 1, 8, 4, [13, 2, 40]),
    (5, "f32", "bf16", 8, 4, 4, 1, [3, 6]),
    (6, "e4m3", "f32", 2, 2, 8, 8, [17, 8, 1]),
])
def test_oracle_matches_brute_force(seed, kv_dtype, q_dtype, hq, hkv, d, p, lens):
    w = custom_workload(len(lens), hq, hkv, d, p, kv_dtype, q_dtype, lens,
                        pool_pages=sum(-(-x // p) for x in lens) + 3)
    case = host_case(w, seed, poison=True)
    out, lse = attention.decode_case(case)
    bo, bl = brute_force(case, w.scale())
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ library

@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 1)])
def test_oracle_matches_torch_sdpa_on_dense_kv(hq, hkv):
    """Identity page table: the result is ordinary attention on dense K/V."""
    rng = np.random.default_rng(11)
    B, D, P = 3, 16, 8
    lens = [37, 8, 1]
    w = custom_workload(B, hq, hkv, D, P, "f32", "f32", lens)
    case = host_case(w, 11, poison=False)
    out, lse = attention.decode_case(case)
    g = hq // hkv
    for r, L in enumerate(lens):
        page, slot = attention.token_locations(case["indptr"], case["indices"],
                                               case["last_page_len"], P, r)
        K = torch.from_numpy(case["kv"][page, 0, slot].astype(np.float64))  # [L, Hkv, D]
        V = torch.from_numpy(case["kv"][page, 1, slot].astype(np.float64))
        Kh = K.permute(1, 0, 2).repeat_interleave(g, dim=0)  # [Hq, L, D]
        Vh = V.permute(1, 0, 2).repeat_interleave(g, dim=0)
        qh = torch.from_numpy(case["q"][r].astype(np.float64))[:, None, :]  # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qh, Kh, Vh, scale=w.scale())
        np.testing.assert_allclose(out[r], ref[:, 0, :].numpy(), rtol=1e-12, atol=1e-12)
        logits = (qh @ Kh.transpose(1, 2))[:, 0, :] * w.scale()
        np.testing.assert_allclose(lse[r], torch.logsumexp(logits, dim=-1).numpy(),
                                   rtol=1e-12, atol=1e-12)
    del rng


# ------------------------------------------------------------------ closed forms

def _case(lens, hq=2, hkv=1, d=8, p=4, dtype="f32", seed=0):
    w = custom_workload(len(lens), hq, hkv, d, p, dtype, "f32", lens,
                        pool_pages=sum(-(-x // p) for x in lens) + 2)
    return host_case(w, seed, poison=True)


def test_single_key_returns_its_value_exactly():
    case = _case([1, 1])
    out, lse = attention.decode_case(case)
    for r in range(2):
        page = case["indices"][case["indptr"][r]]
        for h in range(2):
            assert np.array_equal(out[r, h], case["kv"][page, 1, 0, 0].astype(np.float64))
            s = case["workload"].scale() * float(
                np.dot(case["q"][r, h].astype(np.float64), case["kv"][page, 0, 0, 0].astype(np.float64)))
            assert abs(lse[r, h] - s) < 1e-12


def test_constant_v_returns_v():
    case = _case([13, 5])
    c = np.linspace(-2, 3, 8).astype(np.float32)
    case["kv"][:, 1] = c
    out, _ = attention.decode_case(case)
    np.testing.assert_allclose(out, np.broadcast_to(c.astype(np.float64), out.shape), rtol=0,
                               atol=1e-14)


def test_zero_query_gives_mean_and_log_length():
    case = _case([13, 5, 4])
    case["q"][:] = 0
    out, lse = attention.decode_case(case)
    for r, L in enumerate([13, 5, 4]):
        page, slot = attention.token_locations(case["indptr"], case["indices"],
                                               case["last_page_len"], 4, r)
        mean = case["kv"][page, 1, slot, 0].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[r], np.broadcast_to(mean, out[r].shape), atol=1e-14)
        np.testing.assert_allclose(lse[r], math.log(L), atol=1e-14)


def test_two_keys_sigmoid_weights():
    case = _case([2], hq=1)
    out, _ = attention.decode_case(case)
    page = case["indices"][0]
    q = case["q"][0, 0].astype(np.float64)
    k1, k2 = (case["kv"][page, 0, i, 0].astype(np.float64) for i in (0, 1))
    v1, v2 = (case["kv"][page, 1, i, 0].astype(np.float64) for i in (0, 1))
    s1, s2 = case["workload"].scale() * (q @ k1), case["workload"].scale() * (q @ k2)
    a = 1.0 / (1.0 + math.exp(s2 - s1))
    np.testing.assert_allclose(out[0, 0], a * v1 + (1 - a) * v2, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_page_permutation_invariance_is_bit_exact(dtype):
    w = custom_workload(3, 4, 2, 8, 4, dtype, "bf16", [11, 30, 4], pool_pages=20)
    case = host_case(w, 5, poison=True)
    out, lse = attention.decode_case(case)
    perm = np.random.default_rng(9).permutation(case["num_pages"])  # new id of each page
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    case2 = dict(case)
    case2["kv"] = case["kv"][inv]
    case2["indices"] = perm[case["indices"]].astype(np.int32)
    if dtype == "e4m3":
        case2["k_scale"] = case["k_scale"][inv]
        case2["v_scale"] = case["v_scale"][inv]
    out2, lse2 = attention.decode_case(case2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_unread_slots_never_reach_the_output():
    case = _case([13, 5, 4], dtype="bf16")
    out, lse = attention.decode_case(case)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_gqa_head_mapping_consecutive_groups():
    """Query heads [kvh*g, (kvh+1)*g) must see KV head kvh only."""
    w = custom_workload(1, 6, 3, 4, 4, "f32", "f32", [9], pool_pages=4)
    case = host_case(w, 2, poison=True)
    base, _ = attention.decode_case(case)
    case["kv"][:, :, :, 2] *= 3.0  # change KV head 2 only
    out, _ = attention.decode_case(case)
    assert np.array_equal(out[0, :4], base[0, :4])
    assert not np.allclose(out[0, 4:], base[0, 4:])


# ------------------------------------------------------------------ worked example

def test_worked_page_table_gather_probe():
    """Gather mapping pinned by the pages' two page lists that share a prefix.

    V carries (page, slot) in its first two lanes; for each target token, K and
    q are set so that the target's logit exceeds every other by 1000, which
    drives every other weight to exactly 0 in float64, so the output must
    equal the target's V exactly.
    """
    with open(os.path.join(GOLDEN, "page_table_example.json")) as f:
        ex = json.load(f)
    P = ex["page_size"]
    lists = ex["page_ids"]
    last = ex["last_page_len"]
    table = explicit_table(lists, last, P, num_pages=max(max(x) for x in lists) + 1)
    D = 4
    w = custom_workload(len(lists), 1, 1, D, P, "f32", "f32",
                        [int(x) for x in table["kv_lens"]], pool_pages=table["num_pages"])
    case = host_case(w, 0, poison=True, table=table)
    kv = case["kv"]
    kv[:, :, :, 0, :] = np.where(np.isnan(kv[:, :, :, 0, :]), np.nan, 0.0)
    pages = np.arange(table["num_pages"])[:, None]
    slots = np.arange(P)[None, :]
    readable = ~np.isnan(kv[:, 1, :, 0, 0])
    kv[:, 1, :, 0, 0] = np.where(readable, pages, np.nan)
    kv[:, 1, :, 0, 1] = np.where(readable, slots, np.nan)
    case["q"][:] = 0
    case["q"][:, 0, 0] = 1.0
    gap = 1000.0 / w.scale()
    for r, plist in enumerate(lists):
        L = int(table["kv_lens"][r])
        for t in range(L):
            page, slot = plist[t // P], t % P
            kv[:, 0, :, 0, 0] = np.where(np.isnan(kv[:, 0, :, 0, 0]), np.nan, 0.0)
            kv[page, 0, slot, 0, 0] = gap
            out, _ = attention.decode_case(case, requests=[r])
            assert out[r, 0, 0] == page and out[r, 0, 1] == slot, (r, t)
    # The shared prefix: both requests read identical tokens for the shared pages.
    shared = ex["shared_prefix_pages"]
    assert lists[0][:shared] == lists[1][:shared]


@pytest.mark.parametrize("seed,qd,hq,hkv,p,lens", [
    (11, "bf16", 4, 1, 4, [13, 2, 40]),
    (12, "f32", 8, 2, 8, [17, 8, 1, 33]),
])
def test_rowwise_e4m3_scales_match_brute_force(seed, qd, hq, hkv, p, lens):
    """One scale per (page, slot, KV head): the brute force indexes it by the
    slot it walks to; the oracle by its vectorised gather."""
    w = custom_workload(len(lens), hq, hkv, 8, p, "e4m3", qd, lens,
                        pool_pages=sum(-(-x // p) for x in lens) + 3, kv_scale="token")
    case = host_case(w, seed, poison=True)
    assert case["k_scale"].shape == (case["kv"].shape[0], hkv, p)
    out, lse = attention.decode_case(case)
    bo, bl = brute_force(case, w.scale())
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def test_rowwise_scales_equal_to_page_scales_give_page_results():
    """Per-token scales that repeat each page's scale reproduce the per-page path."""
    w = custom_workload(3, 8, 2, 16, 4, "e4m3", "bf16", [13, 2, 40], pool_pages=20)
    case = host_case(w, 13, poison=True)
    out0, lse0 = attention.decode_case(case)
    P = case["kv"].shape[2]
    tok = dict(case)
    tok["k_scale"] = np.repeat(case["k_scale"][:, :, None], P, axis=2)
    tok["v_scale"] = np.repeat(case["v_scale"][:, :, None], P, axis=2)
    out1, lse1 = attention.decode_case(tok)
    np.testing.assert_array_equal(out0, out1)
    np.testing.assert_array_equal(lse0, lse1)


def test_f16_storage_matches_brute_force():
    w = custom_workload(3, 8, 2, 8, 4, "f16", "f16", [13, 2, 40], pool_pages=20)
    case = host_case(w, 21, poison=True)
    assert case["kv"].dtype == np.float16 and case["q"].dtype == np.float16
    out, lse = attention.decode_case(case)
    bo, bl = brute_force(case, w.scale())
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)
