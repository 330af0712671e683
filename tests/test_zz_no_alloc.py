"""pkd_run_static, the entry point that allocates nothing, against pkd_run.

Two calls in a row on one device, the second with a smaller batch (so the
static scratch still holds the first call's larger work list and partial
states), each compared bit for bit with pkd_run's result on a caller
workspace (same kernels, same launch) and with the oracle. The first plan
splits many requests (separate merge kernel) and has more work units than
one workgroup per compute unit (a persistent launch, whose work counters
live in the scratch), the second few (merge folded into the decode kernel,
whose arrival counters live in the scratch too).
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_plan_amd as pk
from gpu_helpers import compare, oracle_for, to_device, workspace
from workloads import custom_workload, host_case

pytestmark = pytest.mark.gpu


def _run_both(lens, seed, **plan_kw):
    w = custom_workload(len(lens), 32, 8, 128, 16, "bf16", "bf16", lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 7)
    case = host_case(w, seed, poison=True)
    dc = to_device(case)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], w.num_qo_heads, w.num_kv_heads,
            w.head_dim, w.page_size, q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16,
            out_data_type=torch.float32, sm_scale=w.scale(), **plan_kw)
    info = wr.plan_info
    out_s, lse_s = wr.run(dc["q"], dc["kv"], return_lse=True, static_scratch=True)
    torch.cuda.synchronize()
    out_w, lse_w = wr.run(dc["q"], dc["kv"], return_lse=True)
    torch.cuda.synchronize()
    wr.close()
    return case, info, (out_s, lse_s), (out_w, lse_w)


def test_static_scratch_matches_the_workspace_run_twice():
    print("[gpu] no-alloc: first call (many split requests)", flush=True)
    big = [4096] * 12 + [100, 3000, 17, 2500]
    case1, info1, s1, w1 = _run_both(big, 71, slots=256, balance=2, min_chunk_pages=4)
    assert info1["num_split_requests"] >= 12 and info1["merge_folded"] == 0
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert info1["num_items"] * info1["units_per_item"] > cus
    print("[gpu] no-alloc: second call (smaller batch, merge folded)", flush=True)
    small = [900, 33, 2048]
    case2, info2, s2, w2 = _run_both(small, 72, slots=8, balance=1, min_chunk_pages=1)
    assert info2["num_split_requests"] > 0 and info2["merge_folded"] == 1
    assert info2["workspace_bytes"] < info1["workspace_bytes"]
    for case, s, wres in ((case1, s1, w1), (case2, s2, w2)):
        assert torch.equal(s[0], wres[0]) and torch.equal(s[1], wres[1])
        ref, ref_lse = oracle_for(case)
        compare(s[0], s[1], ref, ref_lse, "bf16")


def test_static_scratch_refuses_a_plan_larger_than_the_scratch():
    lens = [2048] * 64
    w = custom_workload(len(lens), 32, 8, 128, 16, "bf16", "bf16", lens, pool_pages=8192 + 3)
    case = host_case(w, 73, poison=False)
    dc = to_device(case)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 32, 8, 128, 16,
            q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16, slots=16384, balance=1,
            min_chunk_pages=1)
    assert wr.plan_info["workspace_bytes"] > 16 << 20
    with pytest.raises(pk.PkdError) as e:
        wr.run(dc["q"], dc["kv"], static_scratch=True)
    assert e.value.code == pk._lib.PKD_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in str(e.value)
    wr.close()
