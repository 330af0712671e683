"""Several new tokens per request (causal within them): HIP path against the oracle.

Each request brings q_r new tokens (its last q_r KV tokens, ragged q rows by
qo_indptr); token i sees the first L_r - q_r + 1 + i KV tokens. A work item
carries up to 16 / group tokens of one request on the MFMA columns. Same
tolerances as the one-token tests; index-exact properties are bit-exact.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import compare, oracle_for, out_to_f64, run_hip, sample_request_case, to_device
from workloads import CONFIGS, custom_workload, device_case, host_case

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 100, 333, 700, 64, 3, 40]
NQ = [1, 5, 16, 3, 7, 2, 9, 4, 3, 30]


def _say(*a):
    print("[gpu-mq]", *a, flush=True)


def _case(kv, g, P=16, lens=LENS, nq=NQ, seed=0, hkv=2):
    nq = [min(a, b) for a, b in zip(nq, lens)]
    w = custom_workload(len(lens), hkv * g, hkv, 128, P, kv, "bf16", lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 5, qo_lens=nq)
    return w, host_case(w, seed, poison=True)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_small_ragged_multi_query_matches_oracle(kv, g, split):
    seed = 300 + g
    w, case = _case(kv, g, seed=seed)
    _say("small", kv, g, split, "seed", seed)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=64, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(to_device(case), **kw)
    assert out.shape == (int(case["qo_indptr"][-1]), w.num_qo_heads, 128)
    max_q = int(np.diff(case["qo_indptr"]).max())
    assert info["queries_per_item"] == (32 // g if max_q * g > 16 else max(1, 16 // g))
    if split == "forced":
        assert info["num_split_requests"] > 0
    compare(out, lse, ref_out, ref_lse, kv)


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "f16"])
@pytest.mark.parametrize("g", [1, 4, 16, 32])
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_two_column_groups(kv, g, split):
    """Items of 17-32 query rows (two 16-column groups sharing every K/V load):
    many new tokens per request, and 32 query heads per KV head."""
    lens, nq = [40, 333, 17, 100, 700], [30, 7, 4, 16, 25]
    if g >= 16:
        nq = [min(x, 5) for x in nq]
    qd = "f16" if kv == "f16" else "bf16"
    w = custom_workload(len(lens), 2 * g, 2, 128, 16, kv, qd, lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 3, qo_lens=nq)
    case = host_case(w, 60 + g, poison=True)
    _say("two groups", kv, g, split)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=32, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(to_device(case), **kw)
    assert info["queries_per_item"] == (32 // g if g < 32 else 1)
    compare(out, lse, ref_out, ref_lse, kv)


def test_group_32_one_token():
    lens = [1, 15, 16, 17, 100, 333, 700]
    w = custom_workload(len(lens), 64, 2, 128, 16, "bf16", "bf16", lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 3)
    case = host_case(w, 77, poison=True)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=16, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "bf16")


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_multi_query_page_sizes(kv, P):
    lens, nq = [1, P + 1, 3 * P + 5, 257, 90], [1, 2, 8, 13, 4]
    w, case = _case(kv, 4, P=P, lens=lens, nq=nq, seed=40 + P)
    _say("pages", kv, P)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, kv)


def test_chunks_past_a_tokens_causal_limit_give_empty_partials():
    """Short chunks of a request whose 30 new tokens span its last two pages:
    the early tokens see nothing of the last chunk, whose partial for them is
    the empty state; the merge must skip it."""
    import paged_kv_decode_plan_amd as pk
    lens, nq = [40, 18], [30, 17]
    w, case = _case("bf16", 4, lens=lens, nq=nq, seed=7)
    kw = dict(slots=64, balance=1, min_chunk_pages=1)
    _, items, _, _ = pk.plan_partition(case["indptr"], case["last_page_len"], 8, 2, 128, 16,
                                       qo_indptr=case["qo_indptr"], **kw)
    assert np.sum(items[:, 7] + items[:, 6] - 1 <= 0) > 0  # blocks that see none of a chunk
    ref_out, ref_lse = oracle_for(case)
    out, lse, info = run_hip(to_device(case), **kw)
    assert info["num_merge_tasks"] >= nq[0]
    compare(out, lse, ref_out, ref_lse, "bf16")


def test_one_token_through_qo_indptr_is_bit_identical_to_plain_decode():
    lens = [5, 300, 17, 64]
    w = custom_workload(4, 16, 4, 128, 16, "bf16", "bf16", lens, pool_pages=40)
    case = host_case(w, 3, poison=True)
    dc = to_device(case)
    out0, lse0, _ = run_hip(dc, slots=8, balance=1, min_chunk_pages=1)
    dc["qo_indptr"] = np.arange(5, dtype=np.int32)
    out1, lse1, _ = run_hip(dc, slots=8, balance=1, min_chunk_pages=1)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_newest_token_row_equals_one_token_decode():
    """The last new token of each request sees the whole request: its row and
    the one-token decode of the same q row both match the oracle's row."""
    lens, nq = [100, 333, 64], [4, 4, 4]
    w, case = _case("bf16", 4, lens=lens, nq=nq, seed=9, hkv=2)
    dc = to_device(case)
    out, lse, _ = run_hip(dc)
    last = case["qo_indptr"][1:] - 1
    one = dict(dc)
    one["q"] = dc["q"][torch.as_tensor(last, device=dc["q"].device)].contiguous()
    one["qo_indptr"] = None
    ref_out, ref_lse = oracle_for(case)
    out1, lse1, _ = run_hip(one)
    compare(out1, lse1, ref_out[last], ref_lse[last], "bf16")
    compare(out[torch.as_tensor(last, device=out.device)], lse[torch.as_tensor(last, device=out.device)],
            ref_out[last], ref_lse[last], "bf16")


def test_full_size_spec4_sampled_requests():
    name = "spec4_llama3_8b_bf16"
    w = CONFIGS[name]
    seed = list(CONFIGS).index(name) + 1
    _say("full-size", name, "seed", seed)
    dc = device_case(w, seed, "cuda:0", poison=True)
    out, lse, info = run_hip(dc)
    _say("plan", info)
    assert info["query_rows"] == 4 * w.batch and info["queries_per_item"] == 4
    o = out_to_f64(out)
    assert np.all(np.isfinite(o))
    qo = dc["qo_indptr"]
    for r in (0, 17, w.batch - 1):
        sub = sample_request_case(dc, r)
        ref_out, ref_lse = oracle_for(sub)
        q0, q1 = int(qo[r]), int(qo[r + 1])
        compare(out[q0:q1], lse[q0:q1], ref_out, ref_lse, "bf16")
    del dc
    torch.cuda.empty_cache()
