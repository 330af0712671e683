"""Pins for the oracle's partition rule: hand-worked cases and invariants."""
import json
import math
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


def _near_equal_table(rng, B, P, N):
    """B requests of at most N pages, each at least N - N // 9 (so the longest is
    within 1/8 of the mean), the first exactly N."""
    n = rng.integers(N - N // 9, N + 1, size=B)
    n[0] = N
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = rng.integers(1, P + 1, size=B).astype(np.int32)
    return indptr, last


def partition_case(seed):
    """A seeded plan() input. Seeds cycle over three kinds so that a third of
    them are near-equal batches, a third single requests (always near-equal),
    and a third free random tables; slots_per_cu is drawn from 1-4."""
    rng = np.random.default_rng(seed)
    P = int(rng.choice([1, 4, 16, 64]))
    kind = seed % 3
    if kind == 0:
        B = int(rng.integers(1, 40))
        indptr, last = _random_table(rng, B, P, int(rng.integers(1, 300)))
    elif kind == 1:
        indptr, last = _near_equal_table(rng, int(rng.integers(2, 300)), P,
                                         int(rng.integers(1, 400)))
    else:
        indptr, last = _near_equal_table(rng, 1, P, int(rng.integers(1, 5000)))
    return dict(indptr=indptr, last=last, P=P, hkv=int(rng.choice([1, 2, 4, 8])),
                slots=int(rng.integers(1, 2048)), balance=int(rng.integers(1, 5)),
                cmin=int(rng.integers(1, 40)), per_cu=int(rng.integers(1, 5)))


def expected_chunk_pages(c):
    """The chunk length the rule asks for, found by enumeration.

    Near-equal batches: every k from 1 to max(1, N // C_min) is priced as
    (equal work units over the compute units, in whole waves) x (one unit's
    pages + 2 C_min), and the cheapest k, the smallest on ties, gives
    C = ceil(N / k). Other batches: the fair share of a slot, clamped to
    [C_min, N]."""
    n = np.diff(c["indptr"]).astype(np.int64)
    B, S, N, H = len(n), int(n.sum()), int(n.max()), c["hkv"]
    if 8 * N * B <= 9 * S:
        cus = math.ceil(c["slots"] / c["per_cu"])
        kmax = max(1, N // c["cmin"])
        prices = {k: math.ceil(B * H * k / (cus * c["balance"])) * (math.ceil(N / k) + 2 * c["cmin"])
                  for k in range(1, kmax + 1)}
        cheapest = min(prices.values())
        k = min(k for k, v in prices.items() if v == cheapest)
        return math.ceil(N / k), True
    share = math.ceil(S * H / (c["slots"] * c["balance"]))
    return min(N, max(c["cmin"], share)), False


def check_partition(seed):
    """Every pin of one seeded partition: the chunk length against the
    enumeration above, then coverage, token counts, partial slots, merge
    index and order checked from their definitions."""
    c = partition_case(seed)
    indptr, last, P = c["indptr"], c["last"], c["P"]
    B = len(last)
    p = oplan.plan(indptr, last, P, c["hkv"], c["slots"], c["balance"], c["cmin"],
                   slots_per_cu=c["per_cu"])
    C = p["chunk_pages"]
    n = np.diff(indptr)
    L = (n - 1) * P + last
    assert C == expected_chunk_pages(c)[0]
    assert 1 <= C <= int(n.max())
    items = p["items"]
    # coverage: per request, chunks tile its page range in order, tokens add up
    for r in range(B):
        mine = items[items[:, 0] == r]
        mine = mine[np.argsort(mine[:, 1])]
        assert mine[0, 1] == indptr[r] and mine[-1, 2] == indptr[r + 1]
        assert np.all(mine[1:, 1] == mine[:-1, 2])
        assert np.all(mine[:, 2] - mine[:, 1] <= C) and np.all(mine[:, 2] > mine[:, 1])
        assert mine[:, 3].sum() == L[r]
        # each chunk's tokens: whole pages, less the tail of the request's last page
        tail = np.where(mine[:, 2] == indptr[r + 1], P - last[r], 0)
        assert np.array_equal(mine[:, 3], (mine[:, 2] - mine[:, 1]) * P - tail)
        G = len(mine)
        assert G == -(-n[r] // C)
        if G > 1:
            assert mine[:, 4].tolist() == list(range(p["merge_indptr"][r], p["merge_indptr"][r] + G))
        else:
            assert mine[0, 4] == -1 and p["merge_indptr"][r + 1] == p["merge_indptr"][r]
    # partial slots are a permutation of [0, num_partials)
    slots_used = np.sort(items[items[:, 4] >= 0, 4])
    assert np.array_equal(slots_used, np.arange(p["num_partials"]))
    # longest first, ties by request, then chunk
    keys = list(zip(-items[:, 3], items[:, 0], items[:, 1]))
    assert keys == sorted(keys)
    assert p["split_requests"].tolist() == [r for r in range(B) if -(-n[r] // C) > 1]


SEEDS = range(90)


@pytest.mark.parametrize("seed", SEEDS)
def test_partition_invariants(seed):
    check_partition(seed)


def test_partition_seeds_reach_both_branches():
    """At least a third of the seeded cases take the near-equal branch, some
    of them with several slots per compute unit and with one request, and the
    enumeration there picks more than one distinct k."""
    near = [s for s in SEEDS if expected_chunk_pages(partition_case(s))[1]]
    assert 3 * len(near) >= len(SEEDS)
    assert any(partition_case(s)["per_cu"] > 1 for s in near)
    assert any(len(partition_case(s)["last"]) == 1 for s in near)
    assert len(near) < len(SEEDS)
    split = [s for s in near
             if expected_chunk_pages(partition_case(s))[0] < np.diff(partition_case(s)["indptr"]).max()]
    assert split and len(split) < len(near)


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


def test_cost_ties_take_the_fewest_chunks():
    """Three requests of 4 pages, one KV head, 2 slots, C_min = 1, worked by
    hand: k=1 costs ceil(3/2)*(4+2) = 12, k=2 ceil(6/2)*(2+2) = 12, k=3
    ceil(9/2)*(2+2) = 20, k=4 ceil(12/2)*(1+2) = 18. k=1 and k=2 tie; the
    smaller k wins, so the requests stay whole (C = 4) rather than C = 2."""
    indptr = np.array([0, 4, 8, 12], np.int32)
    last = np.array([16, 5, 16], np.int32)
    p = oplan.plan(indptr, last, 16, 1, slots=2, balance=1, min_chunk_pages=1)
    assert p["chunk_pages"] == 4 and p["num_partials"] == 0
    # the same batch on 2 compute units with 2 slots each (4 slots) prices
    # waves over compute units: identical choice
    p = oplan.plan(indptr, last, 16, 1, slots=4, balance=1, min_chunk_pages=1, slots_per_cu=2)
    assert p["chunk_pages"] == 4


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
