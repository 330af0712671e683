"""Pins for the oracle's partition rule: hand-worked cases and invariants."""
import json
import os

import numpy as np
import pytest

from oracle import plan as oplan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_partitions():
    with open(os.path.join(GOLDEN, "plan_worked_example.json")) as f:
        ex = json.load(f)
    for c in ex["cases"]:
        p = oplan.plan(c["indptr"], c["last_page_len"], ex["page_size"], ex["num_kv_heads"],
                       c["slots"], c["balance"], c["min_chunk_pages"])
        assert p["chunk_pages"] == c["chunk_pages"], c["work"]
        assert p["items"][:, :5].tolist() == c["items"], c["work"]
        assert p["merge_indptr"].tolist() == c["merge_indptr"], c["work"]
        # one query token per request: its own row, and it sees the whole item
        items = p["items"]
        assert np.array_equal(items[:, 5], items[:, 0])
        assert np.all(items[:, 6] == 1) and np.array_equal(items[:, 7], items[:, 3])


def test_hand_worked_multi_query_partitions():
    with open(os.path.join(GOLDEN, "plan_worked_example.json")) as f:
        ex = json.load(f)
    for c in ex["multi_query_cases"]:
        p = oplan.plan(c["indptr"], c["last_page_len"], ex["page_size"], ex["num_kv_heads"],
                       c["slots"], c["balance"], c["min_chunk_pages"], c["qo_indptr"],
                       c["queries_per_item"])
        assert p["chunk_pages"] == c["chunk_pages"], c["work"]
        assert p["items"].tolist() == c["items"], c["work"]
        assert p["merge_indptr"].tolist() == c["merge_indptr"], c["work"]
        assert p["num_partials"] == c["num_partials"], c["work"]


def _random_table(rng, B, P, max_pages):
    n = rng.integers(1, max_pages + 1, size=B)
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = rng.integers(1, P + 1, size=B).astype(np.int32)
    return indptr, last


@pytest.mark.parametrize("seed", range(25))
def test_partition_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    P = int(rng.choice([1, 4, 16, 64]))
    indptr, last = _random_table(rng, B, P, int(rng.integers(1, 300)))
    hkv = int(rng.choice([1, 2, 8]))
    slots = int(rng.integers(1, 2048))
    balance = int(rng.integers(1, 5))
    cmin = int(rng.integers(1, 40))
    p = oplan.plan(indptr, last, P, hkv, slots, balance, cmin)
    C = p["chunk_pages"]
    n = np.diff(indptr)
    L = (n - 1) * P + last
    S, N = int(n.sum()), int(n.max())
    # chunk length: the closed form, and its bounds
    if 8 * N * B <= 9 * S and 2 * B * hkv >= slots:
        assert C == N
    else:
        assert C == min(N, max(cmin, -(-(S * hkv) // (slots * balance))))
    assert 1 <= C <= N
    items = p["items"]
    # coverage: per request, chunks tile its page range in order, tokens add up
    for r in range(B):
        mine = items[items[:, 0] == r]
        mine = mine[np.argsort(mine[:, 1])]
        assert mine[0, 1] == indptr[r] and mine[-1, 2] == indptr[r + 1]
        assert np.all(mine[1:, 1] == mine[:-1, 2])
        assert np.all(mine[:, 2] - mine[:, 1] <= C) and np.all(mine[:, 2] > mine[:, 1])
        assert mine[:, 3].sum() == L[r]
        G = len(mine)
        assert G == -(-n[r] // C)
        if G > 1:
            assert mine[:, 4].tolist() == list(range(p["merge_indptr"][r], p["merge_indptr"][r] + G))
        else:
            assert mine[0, 4] == -1 and p["merge_indptr"][r + 1] == p["merge_indptr"][r]
    # partial slots are a permutation of [0, num_partials)
    slots_used = np.sort(items[items[:, 4] >= 0, 4])
    assert np.array_equal(slots_used, np.arange(p["num_partials"]))
    # longest first, ties by request
    keys = list(zip(-items[:, 3], items[:, 0], items[:, 1]))
    assert keys == sorted(keys)
    assert p["split_requests"].tolist() == [r for r in range(B) if -(-n[r] // C) > 1]


@pytest.mark.parametrize("seed", range(25))
def test_multi_query_partition_invariants(seed):
    """Every new token of every request sees each of its pages through exactly one
    item, with the causal token count; partial rows are a permutation."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 20))
    P = int(rng.choice([1, 4, 16]))
    indptr, last = _random_table(rng, B, P, int(rng.integers(1, 60)))
    n = np.diff(indptr)
    L = (n - 1) * P + last
    nq = np.minimum(rng.integers(1, 12, size=B), L)
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    Q = int(rng.integers(1, 9))
    hkv = int(rng.choice([1, 2, 8]))
    p = oplan.plan(indptr, last, P, hkv, int(rng.integers(1, 512)), int(rng.integers(1, 4)),
                   int(rng.integers(1, 10)), qo, Q)
    C = p["chunk_pages"]
    items = p["items"]
    U = -(-nq // Q)
    units, S = int(U.sum()), int((n * U).sum())
    assert len(items) == int((-(-n // C) * U).sum())
    rows_written = []
    for r in range(B):
        for j in range(int(nq[r])):
            row = int(qo[r]) + j
            mine = items[(items[:, 0] == r) & (items[:, 5] <= row) & (row < items[:, 5] + items[:, 6])]
            mine = mine[np.argsort(mine[:, 1])]
            assert mine[0, 1] == indptr[r] and mine[-1, 2] == indptr[r + 1]
            assert np.all(mine[1:, 1] == mine[:-1, 2])
            own = int(L[r] - nq[r] + j)  # position of this token in its request
            for it in mine:
                i = row - it[5]
                first_tok = (it[1] - indptr[r]) * P
                seen = sum(1 for t in range(first_tok, first_tok + it[3]) if t <= own)
                assert max(0, min(it[3], it[7] + i)) == seen
                if it[4] >= 0:
                    rows_written.append(int(it[4]) + i)
    assert sorted(rows_written) == list(range(p["num_partials"]))
    G = -(-n // C)
    assert p["merge_indptr"].tolist() == np.concatenate(
        [[0], np.cumsum(np.where(G > 1, G * nq, 0))]).tolist()
    keys = [(-it[3], it[0], it[1], it[5]) for it in items]
    assert keys == sorted(keys)


def test_uniform_batch_is_cut_to_fill_the_device():
    """Near-equal requests: k chunks per request minimising
    ceil(units * k / CUs) * (ceil(N / k) + 2 * C_min), worked by hand."""
    indptr = np.arange(0, 65 * 4, 4, dtype=np.int32)  # 64 requests of 4 pages
    last = np.full(64, 16, np.int32)
    # 512 units, 512 slots: k=1 costs 1*(4+2)=6, k=2 2*(2+2)=8, k=3 3*4=12, k=4 4*3=12 -> whole
    p = oplan.plan(indptr, last, 16, 8, slots=512, balance=1, min_chunk_pages=1)
    assert p["chunk_pages"] == 4 and p["num_partials"] == 0
    # 1024 slots: 6, 1*4=4, 2*4=8, 2*3=6 -> k=2, C=2: every request in two chunks
    p = oplan.plan(indptr, last, 16, 8, slots=1024, balance=1, min_chunk_pages=1)
    assert p["chunk_pages"] == 2 and p["num_partials"] == 128
    # 2048 slots: 6, 4, 1*4=4, 1*3=3 -> k=4, C=1
    p = oplan.plan(indptr, last, 16, 8, slots=2048, balance=1, min_chunk_pages=1)
    assert p["chunk_pages"] == 1 and p["num_partials"] == 256
    # C_min bounds k: with C_min=4 only k=1 is allowed
    p = oplan.plan(indptr, last, 16, 8, slots=2048, balance=1, min_chunk_pages=4)
    assert p["chunk_pages"] == 4 and p["num_partials"] == 0


def test_waves_count_compute_units_not_slots():
    # 512 units, 1024 slots at 4 per CU = 256 CUs: k=1 costs 2*(4+2)=12,
    # k=2 4*(2+2)=16, k=3 6*4=24, k=4 8*3=24 -> whole (every CU already busy)
    indptr = np.arange(0, 65 * 4, 4, dtype=np.int32)
    last = np.full(64, 16, np.int32)
    p = oplan.plan(indptr, last, 16, 8, slots=1024, balance=1, min_chunk_pages=1,
                   slots_per_cu=4)
    assert p["chunk_pages"] == 4 and p["num_partials"] == 0


def test_uniform_batch_just_over_the_device_is_cut_into_waves():
    # 72 requests of 128 pages, 4 units each = 288 units on 256 slots, C_min=16:
    # k=1: 2*(128+32)=320; k=2: 3*(64+32)=288; k=3: 4*(43+32)=300;
    # k=4: 5*(32+32)=320; k=5: 6*(26+32)=348; k=6: 7*(22+32)=378;
    # k=7: 8*(19+32)=408; k=8: 9*(16+32)=432 -> k=2, C=64
    indptr = np.arange(0, 73 * 128, 128, dtype=np.int32)
    last = np.full(72, 16, np.int32)
    p = oplan.plan(indptr, last, 16, 4, slots=256, balance=1, min_chunk_pages=16)
    assert p["chunk_pages"] == 64 and p["num_partials"] == 72 * 2


def test_unequal_batch_is_split_even_with_enough_units():
    indptr = np.concatenate([[0], np.cumsum([128] * 63 + [300])]).astype(np.int32)
    last = np.full(64, 16, np.int32)
    p = oplan.plan(indptr, last, 16, 8, slots=1024, balance=1, min_chunk_pages=16)
    assert p["chunk_pages"] < 300 and p["num_partials"] > 0


@pytest.mark.parametrize("bad", [
    dict(indptr=[0, 0], last=[1]),      # empty request
    dict(indptr=[0, 2], last=[0]),      # last_page_len below 1
    dict(indptr=[0, 2], last=[17]),     # above page_size
    dict(indptr=[1, 2], last=[1]),      # indptr[0] != 0
])
def test_invalid_tables_rejected(bad):
    with pytest.raises(ValueError):
        oplan.plan(bad["indptr"], bad["last"], 16, 1, 8, 1, 1)


def test_non_causal_rows_see_every_item_token():
    """The shared-prefix level of cascade attention: rows are not causal, and a
    request may carry more query rows than it has KV tokens."""
    indptr, last = [0, 3, 4], [3, 2]
    p = oplan.plan(indptr, last, 4, 1, 8, 1, 1, qo_indptr=[0, 20, 23], queries_per_item=4,
                   causal=False)
    items = p["items"]
    assert np.array_equal(items[:, 7], items[:, 3])
    with pytest.raises(ValueError):  # 3 rows over 2 tokens is only legal without causality
        oplan.plan(indptr, last, 4, 1, 8, 1, 1, qo_indptr=[0, 20, 23], queries_per_item=4)
    for r, (q0, q1) in enumerate([(0, 20), (20, 23)]):
        for row in range(q0, q1):
            mine = items[(items[:, 0] == r) & (items[:, 5] <= row) & (row < items[:, 5] + items[:, 6])]
            assert sorted(mine[:, 1].tolist()) == sorted(set(mine[:, 1].tolist()))
            assert mine[:, 3].sum() == (indptr[r + 1] - indptr[r] - 1) * 4 + last[r]
