"""The C++ planner (through the C ABI, host only) against the oracle's rule, bit for bit."""
import json
import os

import numpy as np
import pytest

import paged_kv_decode_plan_amd as pk
from oracle import plan as oplan
from workloads import CONFIGS, page_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _both(indptr, last, P, hkv, slots, balance, cmin, hq=None, d=128, kv="bf16",
          qo_indptr=None, qd=None):
    hq = hq or hkv
    qd = qd or ("f16" if kv == "f16" else "bf16")
    info, items, merge, split = pk.plan_partition(indptr, last, hq, hkv, d, P, kv_dtype=kv,
                                                  q_dtype=qd, slots=slots, balance=balance,
                                                  min_chunk_pages=cmin, qo_indptr=qo_indptr)
    ref = oplan.plan(indptr, last, P, info["units_per_item"], slots, balance, cmin, qo_indptr,
                     info["queries_per_item"])
    return info, items, merge, split, ref


def _assert_same(info, items, merge, split, ref):
    assert info["chunk_pages"] == ref["chunk_pages"]
    assert np.array_equal(items, ref["items"])
    assert np.array_equal(merge, ref["merge_indptr"])
    assert np.array_equal(split, ref["split_requests"])
    assert info["num_partials"] == ref["num_partials"]
    assert info["total_kv_tokens"] == int(ref["kv_lens"].sum())


def test_golden_partitions_native():
    with open(os.path.join(GOLDEN, "plan_worked_example.json")) as f:
        ex = json.load(f)
    for c in ex["cases"]:
        info, items, merge, split, ref = _both(c["indptr"], c["last_page_len"], ex["page_size"],
                                               1, c["slots"], c["balance"], c["min_chunk_pages"])
        assert items[:, :5].tolist() == c["items"]
        _assert_same(info, items, merge, split, ref)


def expected_queries_per_item(max_q: int, g: int, kv: str) -> int:
    """One token per request: 1; else a 16-row column group of tokens, or two
    (32 rows) when the tokens need more than one and the form has them."""
    if max_q == 1:
        return 1
    if max_q * g > 16 and kv != "e2m1":
        return 32 // g
    return max(1, 16 // g)


def test_golden_multi_query_partitions_native():
    """Eight query heads per KV head over e2m1 KV (one 16-row column group per
    item): a work item carries 16 / 8 = 2 new tokens."""
    with open(os.path.join(GOLDEN, "plan_worked_example.json")) as f:
        ex = json.load(f)
    for c in ex["multi_query_cases"]:
        info, items, merge, split, ref = _both(
            c["indptr"], c["last_page_len"], ex["page_size"], 1, c["slots"], c["balance"],
            c["min_chunk_pages"], hq=8, qo_indptr=c["qo_indptr"], kv="e2m1")
        assert info["queries_per_item"] == c["queries_per_item"]
        assert items.tolist() == c["items"]
        assert info["num_partials"] == c["num_partials"]
        assert info["query_rows"] == c["qo_indptr"][-1]
        _assert_same(info, items, merge, split, ref)


@pytest.mark.parametrize("seed", range(30))
def test_random_multi_query_tables_bit_exact(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 120))
    P = int(rng.choice([1, 16, 64]))
    n = rng.integers(1, int(rng.integers(2, 200)), size=B)
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = rng.integers(1, P + 1, size=B).astype(np.int32)
    L = (n - 1) * P + last
    nq = np.minimum(rng.integers(1, int(rng.integers(2, 40)), size=B), L)
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    kv = str(rng.choice(["bf16", "e4m3", "e2m1"]))
    out = _both(indptr, last, P, hkv, int(rng.integers(1, 4096)), int(rng.integers(1, 4)),
                int(rng.integers(1, 32)), hq=hkv * g, kv=kv, qo_indptr=qo)
    info = out[0]
    assert info["queries_per_item"] == expected_queries_per_item(int(nq.max()), g, kv)
    assert info["max_qo_len"] == nq.max() and info["query_rows"] == qo[-1]
    _assert_same(*out[:4], out[4])


def test_multi_query_needs_the_mfma_path():
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 2], [5], 4, 4, 64, 16, q_dtype="bf16", qo_indptr=[0, 2])
    assert e.value.code == pk._lib.PKD_ERR_UNSUPPORTED
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 2], [5], 4, 4, 128, 16, kv_dtype="f32", qo_indptr=[0, 2])
    assert e.value.code == pk._lib.PKD_ERR_UNSUPPORTED
    # one token per request through qo_indptr is plain decode: any kernel
    info, items, *_ = pk.plan_partition([0, 2], [5], 4, 4, 64, 16, kv_dtype="f32",
                                        qo_indptr=[0, 1])
    assert info["queries_per_item"] == 1 and items[0, 6] == 1


@pytest.mark.parametrize("qo", [[0, 0, 2], [0, 2, 1], [1, 2, 3], [0, 30, 31]])
def test_invalid_query_layouts_rejected_natively(qo):
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 2, 3], [5, 3], 8, 2, 128, 16, qo_indptr=qo)
    assert e.value.code == pk._lib.PKD_ERR_INVALID_ARGUMENT

@pytest.mark.parametrize("seed", range(40))
def test_random_tables_bit_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 300))
    P = int(rng.choice([1, 2, 16, 64]))
    n = rng.integers(1, int(rng.integers(2, 500)), size=B)
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = rng.integers(1, P + 1, size=B).astype(np.int32)
    hkv = int(rng.choice([1, 2, 4, 8]))
    out = _both(indptr, last, P, hkv, int(rng.integers(1, 4096)), int(rng.integers(1, 6)),
                int(rng.integers(1, 64)), hq=hkv * int(rng.choice([1, 2, 4, 8])))
    _assert_same(*out[:4], out[4])


@pytest.mark.parametrize("name", list(CONFIGS))
@pytest.mark.parametrize("slots", [1024, 2048, 768])
def test_workload_tables_bit_exact(name, slots):
    w = CONFIGS[name]
    t = page_table(w, seed=list(CONFIGS).index(name) + 1)
    cmin = max(1, -(-256 // w.page_size))
    out = _both(t["indptr"], t["last_page_len"], w.page_size, w.num_kv_heads, slots, 2, cmin,
                hq=w.num_qo_heads, d=w.head_dim, kv=w.kv_dtype, qo_indptr=t["qo_indptr"],
                qd=w.q_dtype)
    _assert_same(*out[:4], out[4])


def test_default_balance_and_min_chunk():
    info, *_ = pk.plan_partition([0, 5, 9], [16, 7], 4, 1, 128, 16, slots=8)
    assert info["balance"] == 1 and info["min_chunk_pages"] == 4
    info, *_ = pk.plan_partition([0, 5, 9], [16, 7], 4, 1, 128, 64, slots=8)
    assert info["min_chunk_pages"] == 1
    info, *_ = pk.plan_partition([0, 5, 9], [1, 1], 4, 1, 128, 1, slots=8)
    assert info["min_chunk_pages"] == 64


def _layout_bytes(items, tasks, parts_rows, hkv, d=128):
    """[counts 256 | items 32 B | merge tasks 16 B | fused-merge records 16 B |
    counters 4 B per KV head | partial (m, d) 8 B | partial o 4*D B], each
    region 256-byte aligned."""
    a = lambda x: (x + 255) // 256 * 256
    end = a(256 + items * 32)
    end = a(end + tasks * 16)
    end = a(end + tasks * 16)
    end = a(end + tasks * hkv * 4)
    end = a(end + parts_rows * 8)
    return a(end + parts_rows * d * 4)


def test_workspace_size_formula():
    info, items, merge, split = pk.plan_partition([0, 5, 9], [16, 7], 32, 8, 128, 16, slots=64,
                                                  balance=1, min_chunk_pages=1)
    assert info["num_split_requests"] == 2 and info["num_partials"] > 0
    assert info["num_merge_tasks"] == info["num_split_requests"]
    assert info["workspace_bytes"] == _layout_bytes(info["num_items"], info["num_merge_tasks"],
                                                    info["num_partials"] * 32, 8)
    # several new tokens: one merge task and one partial row per token of a split request
    info, items, merge, split = pk.plan_partition([0, 5, 9], [16, 7], 32, 8, 128, 16, slots=64,
                                                  balance=1, min_chunk_pages=1,
                                                  qo_indptr=[0, 3, 5])
    assert info["num_merge_tasks"] == 5 and info["queries_per_item"] == 4
    assert info["workspace_bytes"] == _layout_bytes(info["num_items"], info["num_merge_tasks"],
                                                    info["num_partials"] * 32, 8)
    # fixed capacity: the layout follows the capacities, not the plan
    cap = dict(items=100, merge_tasks=40, partials=300, qo_len=4)
    info2, *_ = pk.plan_partition([0, 5, 9], [16, 7], 32, 8, 128, 16, slots=64, balance=1,
                                  min_chunk_pages=1, qo_indptr=[0, 3, 5], capacity=cap)
    assert info2["workspace_bytes"] == _layout_bytes(100, 40, 300 * 32, 8)


def test_capacity_limits_are_enforced():
    cap = dict(items=4, merge_tasks=40, partials=300, qo_len=1)
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 5, 9], [16, 7], 32, 8, 128, 16, slots=64, balance=1,
                          min_chunk_pages=1, capacity=cap)
    assert "capacities" in str(e.value)
    with pytest.raises(pk.PkdError):  # more new tokens than capacity_qo_len
        pk.plan_partition([0, 5, 9], [16, 7], 32, 8, 128, 16, qo_indptr=[0, 3, 5],
                          capacity=dict(items=100, merge_tasks=40, partials=300, qo_len=2))
    with pytest.raises(pk.PkdError):  # all four or none
        pk.plan_partition([0, 5, 9], [16, 7], 32, 8, 128, 16, capacity=(100, 0, 300, 1))


@pytest.mark.parametrize("seed", range(20))
def test_item_count_bound_for_capacities(seed):
    """The bound the header gives for capacity_items: query blocks + slots *
    balance / num_kv_heads."""
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 200))
    n = rng.integers(1, int(rng.integers(2, 400)), size=B)
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = rng.integers(1, 17, size=B).astype(np.int32)
    hkv, slots, bal = int(rng.choice([1, 2, 8])), int(rng.integers(1, 3000)), int(rng.integers(1, 4))
    info, items, *_ = pk.plan_partition(indptr, last, 4 * hkv, hkv, 128, 16, slots=slots,
                                        balance=bal, min_chunk_pages=int(rng.integers(1, 20)))
    assert info["num_items"] <= B + slots * bal // info["units_per_item"]


@pytest.mark.parametrize("seed", range(10))
def test_non_causal_tables_bit_exact(seed):
    """The shared-prefix level of cascade attention: many q rows per request,
    more than its tokens allowed, every row sees the whole item."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 6))
    P = 16
    n = rng.integers(1, 300, size=B)
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = rng.integers(1, P + 1, size=B).astype(np.int32)
    nq = rng.integers(1, 200, size=B)
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    g = int(rng.choice([1, 4, 8]))
    info, items, merge, split = pk.plan_partition(indptr, last, 8 * g, 8, 128, P, slots=1024,
                                                  balance=1, min_chunk_pages=16, qo_indptr=qo,
                                                  causal=False)
    ref = oplan.plan(indptr, last, P, info["units_per_item"], 1024, 1, 16, qo,
                     info["queries_per_item"], causal=False)
    _assert_same(info, items, merge, split, ref)
    assert np.array_equal(items[:, 7], items[:, 3])


@pytest.mark.parametrize("q,kv,d", [("bf16", "f16", 128), ("f16", "bf16", 128),
                                    ("f16", "f16", 64), ("f32", "f16", 128)])
def test_fp16_needs_fp16_q_over_fp16_kv_at_128(q, kv, d):
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 2], [5], 8, 2, d, 16, kv_dtype=kv, q_dtype=q)
    assert e.value.code == pk._lib.PKD_ERR_UNSUPPORTED


@pytest.mark.parametrize("q,d", [("f32", 128), ("f16", 128), ("bf16", 64)])
def test_e2m1_needs_bf16_q_at_128(q, d):
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 2], [5], 8, 2, d, 16, kv_dtype="e2m1", q_dtype=q)
    assert e.value.code == pk._lib.PKD_ERR_UNSUPPORTED


def test_e2m1_has_no_row_wise_scales():
    with pytest.raises(pk.PkdError) as e:
        pk.plan_partition([0, 2], [5], 8, 2, 128, 16, kv_dtype="e2m1", q_dtype="bf16",
                          kv_scale="token")
    assert e.value.code == pk._lib.PKD_ERR_INVALID_ARGUMENT


def test_e2m1_plans_match_the_oracle():
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 3000, size=37)
    P = 16
    npg = -(-lens // P)
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    last = (lens - (npg - 1) * P).astype(np.int32)
    for g in (1, 4, 16):
        _assert_same(*_both(indptr, last, P, 8, 256, 1, 16, hq=8 * g, kv="e2m1"))


@pytest.mark.parametrize("hkv,g,P,qo,want_e2m1,want_e4m3", [
    (8, 4, 16, None, 4, 4),     # pairs of KV heads: 4 workgroups per item
    (2, 8, 16, None, 1, 1),
    (3, 4, 16, None, 3, 3),     # odd KV head count: one head per workgroup
    (2, 16, 16, None, 2, 1),    # 2 x 16 rows: two column groups (not for e2m1)
    (8, 4, 8, None, 8, 8),      # pages below 16 tokens
    (8, 4, 16, [0, 2, 3], 4, 4),   # two new tokens: 8 rows per head, pairs
    (8, 4, 16, [0, 9, 10], 8, 8),  # more than 16 rows per head: one head
])
@pytest.mark.parametrize("kv", ["e2m1", "i4", "e4m3"])
def test_head_pair_workgroups_per_item(kv, hkv, g, P, qo, want_e2m1, want_e4m3):
    info, *_ = pk.plan_partition([0, 3, 5], [5, P], hkv * g, hkv, 128, P, kv_dtype=kv,
                                 q_dtype="bf16", qo_indptr=qo)
    assert info["units_per_item"] == (want_e2m1 if kv in ("e2m1", "i4") else want_e4m3)


def test_many_split_workgroups_keep_the_merge_kernel():
    """The merge folds into the decode kernel only for a few split workgroups
    (each pays device-scope fences); a batch of split requests keeps the
    separate merge kernel."""
    P = 16
    few = pk.plan_partition([0, 32], [16], 4, 4, 64, P, kv_dtype="f32", q_dtype="f32",
                            slots=1024, min_chunk_pages=16)[0]
    assert few["num_split_requests"] == 1 and few["merge_folded"] == 1
    indptr = np.arange(0, 64 * 32 + 1, 32, dtype=np.int32)
    many = pk.plan_partition(indptr, [16] * 64, 32, 8, 128, P, kv_dtype="bf16", q_dtype="bf16",
                             slots=1024, min_chunk_pages=16)[0]
    assert many["num_split_requests"] == 64 and many["merge_folded"] == 0


@pytest.mark.parametrize("chunks,folded", [(8, 1), (16, 1), (17, 0)])
def test_fold_takes_up_to_sixteen_chunks(chunks, folded):
    """A split request of up to sixteen chunks over few workgroups folds its
    merge into the decode kernel; one more chunk keeps the merge kernel. The
    single-sequence shape (512 tokens, four KV heads, 64-token chunks) is the
    eight-chunk case."""
    P = 16
    hkv = 4 if chunks == 8 else 1
    info = pk.plan_partition([0, 4 * chunks], [P], hkv, hkv, 64, P, kv_dtype="f32",
                             q_dtype="f32", slots=1024)[0]
    assert info["min_chunk_pages"] == 4 and info["chunk_pages"] == 4
    assert info["num_split_requests"] == 1 and info["merge_folded"] == folded


def test_plans_from_many_threads_match_sequential_plans():
    """pkd_plan_create / get_worklist / destroy from eight host threads at
    once (each with its own tables, and some calls failing on purpose so
    that the thread-local error message is exercised) give the same work
    lists as the same calls made one after another."""
    import threading

    from paged_kv_decode_plan_amd import _lib

    rng = np.random.default_rng(2026)
    cases = []
    for _ in range(64):
        B = int(rng.integers(1, 40))
        P = int(rng.choice([1, 4, 16, 64]))
        lens = rng.integers(1, 3000, B)
        npg = -(-lens // P)
        indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
        last = (lens - (npg - 1) * P).astype(np.int32)
        cases.append((indptr, last, P, int(rng.choice([64, 256, 1024]))))

    def build(c):
        indptr, last, P, slots = c
        info, items, merge, split = pk.plan_partition(indptr, last, 32, 8, 128, P, slots=slots)
        return info["num_items"], items.tobytes(), merge.tobytes(), split.tobytes()

    want = [build(c) for c in cases]
    got = [None] * len(cases)
    errors = []

    def worker(t):
        try:
            for i in range(t, len(cases), 8):
                with pytest.raises(_lib.PkdError, match="indptr"):
                    pk.plan_partition([1, 3], [4], 32, 8, 128, 16)  # indptr[0] != 0
                got[i] = build(cases[i])
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    assert got == want
