"""Persistent decode launches: a plan with more work units (item x KV-head
pair) than the device holds resident workgroups runs as that many
workgroups, each taking units from a counter in the workspace, which the last
one to finish resets. Checked on the GPU against the oracle, and run again
(also after another plan used the same workspace) with identical bits, which
needs the counters back at zero after every launch; one case also folds the
merge of its split requests into the same persistent launch."""
import numpy as np
import pytest
import torch

import paged_kv_decode_plan_amd as pk
from gpu_helpers import compare, oracle_for, run_hip, to_device, workspace
from workloads import custom_workload, host_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-persistent]", *a, flush=True)


def _plan(dc, w, **kw):
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], w.num_qo_heads, w.num_kv_heads,
            w.head_dim, w.page_size, q_data_type=torch.bfloat16,
            kv_data_type="e4m3" if w.kv_dtype == "e4m3" else torch.bfloat16,
            out_data_type=torch.float32, sm_scale=w.scale(), **kw)
    return wr


def _run(wr, dc):
    out, lse = wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                      v_scale=dc["v_scale"])
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("split", ["none", "some", "folded"])
def test_many_units_match_the_oracle_and_repeat(kv, split):
    rng = np.random.default_rng(77 if kv == "bf16" else 78)
    lens = rng.integers(1, 400, size=320).tolist()
    if split == "some":
        lens[:6] = [6000, 5000, 4200, 3900, 3100, 2500]
    elif split == "folded":  # two requests split over few workgroups: the merge folds in
        lens[:2] = [4000, 3500]
    w = custom_workload(len(lens), 32, 8, 128, 16, kv, "bf16", lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 9)
    case = host_case(w, 2024, poison=True)
    dc = to_device(case)
    kw = dict(balance=4) if split == "some" else {}
    wr = _plan(dc, w, **kw)
    info = wr.plan_info
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _say(kv, split, {k: info[k] for k in ("num_items", "units_per_item", "num_split_requests")})
    # more units than one workgroup per compute unit: the persistent launch
    assert info["num_items"] * info["units_per_item"] > 2 * cus
    if split != "none":
        assert info["num_split_requests"] > 0
    assert info["merge_folded"] == (1 if split == "folded" else 0)
    out, lse = _run(wr, dc)
    ref, ref_lse = oracle_for(case)
    compare(out, lse, ref, ref_lse, kv)
    for _ in range(2):
        again, again_lse = _run(wr, dc)
        assert torch.equal(again, out) and torch.equal(again_lse, lse)
    wr.close()

    # another plan through the same workspace (its own upload), then this one again
    small = custom_workload(3, 32, 8, 128, 16, kv, "bf16", [100, 900, 17], pool_pages=70)
    scase = host_case(small, 5, poison=True)
    sdc = to_device(scase)
    swr = _plan(sdc, small, slots=8, balance=1, min_chunk_pages=1)
    sout, slse = _run(swr, sdc)
    sref, sref_lse = oracle_for(scase)
    compare(sout, slse, sref, sref_lse, kv)
    swr.close()
    wr = _plan(dc, w, **kw)
    again, again_lse = _run(wr, dc)
    assert torch.equal(again, out) and torch.equal(again_lse, lse)
    wr.close()


@pytest.mark.parametrize("kv,q_dtype,hq,qo", [
    ("f16", "f16", 32, None),    # fp16 KV on the fp16 MFMA
    ("bf16", "bf16", 32, 3),     # three new tokens per request (12 rows per KV head)
    ("bf16", "bf16", 128, None),  # 16 query heads per KV head: a pair's 32 rows, two column groups
    ("e4m3", "bf16", 32, 2),
])
def test_persistent_launch_other_forms(kv, q_dtype, hq, qo):
    """Persistent launches of the other MFMA forms (fp16 KV, several new
    tokens per request, two column groups per workgroup) against the oracle,
    and bit-identical when run again."""
    rng = np.random.default_rng(90 + hq + (qo or 0))
    lens = rng.integers(4, 300, size=300).tolist()
    qo_lens = None if qo is None else [min(qo, n) for n in lens]
    w = custom_workload(len(lens), hq, 8, 128, 16, kv, q_dtype, lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 9, qo_lens=qo_lens)
    case = host_case(w, 2100 + hq, poison=True)
    dc = to_device(case)
    out, lse, info = run_hip(dc)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _say(kv, q_dtype, hq, qo, {k: info[k] for k in ("num_items", "units_per_item", "slots")})
    assert info["num_items"] * info["units_per_item"] > info["slots"] >= cus
    ref, ref_lse = oracle_for(case)
    compare(out, lse, ref, ref_lse, kv)
    again, again_lse, _ = run_hip(dc)
    assert torch.equal(again, out) and torch.equal(again_lse, lse)


def test_two_persistent_launches_on_two_streams():
    """Two plans with more work units than resident workgroups, each with its
    own workspace and stream (default priority), launched interleaved so that
    the two persistent grids share the device: neither has all its workgroups
    resident, which is safe because no workgroup waits for another (units come
    from a counter that only grows; the last arrival of a split request folds
    its merge). The results equal the same runs made one after the other, bit
    for bit, and the oracle."""
    cases = []
    for seed, (kv, extra) in enumerate([("bf16", None), ("e4m3", [4000, 3500])]):
        rng = np.random.default_rng(90 + seed)
        lens = rng.integers(1, 400, size=320).tolist()
        if extra:
            lens[:len(extra)] = extra
        w = custom_workload(len(lens), 32, 8, 128, 16, kv, "bf16", lens,
                            pool_pages=sum(-(-x // 16) for x in lens) + 5)
        cases.append((w, host_case(w, 300 + seed, poison=True)))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dcs = [to_device(c) for _, c in cases]
    seq = []
    for (w, _), dc in zip(cases, dcs):
        wr = _plan(dc, w)
        info = wr.plan_info
        _say("two streams", w.kv_dtype, {k: info[k] for k in ("num_items", "merge_folded")})
        assert info["num_items"] * info["units_per_item"] > 2 * cus
        seq.append(_run(wr, dc))
        wr.close()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wrappers = []
    for (w, _), dc, st in zip(cases, dcs, streams):
        wr = pk.BatchDecodeWithPagedKVCacheWrapper(
            torch.empty(16 << 20, dtype=torch.uint8, device="cuda:0"), "NHD")
        with torch.cuda.stream(st):
            wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, q_data_type=torch.bfloat16,
                    kv_data_type="e4m3" if w.kv_dtype == "e4m3" else torch.bfloat16,
                    out_data_type=torch.float32, sm_scale=w.scale())
        wrappers.append(wr)
    assert wrappers[1].plan_info["merge_folded"] == 1
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        res = []
        for wr, dc, st in zip(wrappers, dcs, streams):
            with torch.cuda.stream(st):
                res.append(wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                                  v_scale=dc["v_scale"]))
        outs.append(res)
    torch.cuda.synchronize()
    for res in outs:
        for (o, l), (so, sl) in zip(res, seq):
            assert torch.equal(o, so) and torch.equal(l, sl)
    for (w, c), (o, l) in zip(cases, seq):
        ref, ref_lse = oracle_for(c)
        compare(o, l, ref, ref_lse, w.kv_dtype)
    for wr in wrappers:
        wr.close()
