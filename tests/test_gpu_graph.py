"""Fixed-capacity plans and HIP graphs.

A fixed-capacity plan launches grids and kernel arguments that depend only on
its capacities, so run() captured once in a HIP graph computes every later
plan uploaded to the same workspace. Each replay is checked against the
oracle, with eager work in between; fixed-capacity and exact plans of the same
batch agree bit for bit.
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_plan_amd as pk
from gpu_helpers import compare, run_hip, to_device, workspace
from oracle import attention
from workloads import custom_workload, explicit_table, host_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CAP = dict(items=512, merge_tasks=256, partials=1024, qo_len=4)


def _say(*a):
    print("[gpu-graph]", *a, flush=True)


@pytest.mark.parametrize("kv,qd", [("bf16", "bf16"), ("e4m3", "bf16"), ("f32", "f32")])
def test_fixed_capacity_plan_is_bit_identical_to_exact(kv, qd):
    """Same work list, same kernels: a fixed-capacity plan and an exact plan
    whose decode and merge stages run apart give the same bits (an exact
    plan's run() may fold a short merge into the decode kernel, which folds
    in another order: compared within tolerance)."""
    lens = [1, 17, 300, 64, 1000]
    w = custom_workload(5, 16, 4, 128, 16, kv, qd, lens, pool_pages=120)
    case = host_case(w, 4, poison=True)
    dc = to_device(case)
    ref_out, ref_lse = attention.decode_case(case)
    kvt = "e4m3" if kv == "e4m3" else dc["kv"].dtype
    for kw in ({}, dict(slots=16, balance=1, min_chunk_pages=1)):
        res = []
        for cap in (None, dict(CAP, qo_len=1)):
            wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
            wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 16, 4, 128, 16,
                    q_data_type=dc["q"].dtype, kv_data_type=kvt, out_data_type=torch.float32,
                    sm_scale=w.scale(), capacity=cap, **kw)
            out = torch.empty(dc["q"].shape, dtype=torch.float32, device=DEV)
            lse = torch.empty(dc["q"].shape[:2], dtype=torch.float32, device=DEV)
            for st in (pk._lib.STAGE_DECODE, pk._lib.STAGE_MERGE):
                wr.run(dc["q"], dc["kv"], out=out, lse=lse, k_scale=dc["k_scale"],
                       v_scale=dc["v_scale"], stages=st)
            o3, l3 = wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                            v_scale=dc["v_scale"])
            torch.cuda.synchronize()
            compare(o3, l3, ref_out, ref_lse, kv)
            wr.close()
            res.append((out, lse))
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def _tables(rng, pool, P, B, max_len, nq_max):
    lens = rng.integers(1, max_len, size=B)
    n = (lens + P - 1) // P
    pages = rng.permutation(pool)[: int(n.sum())]
    lists, at = [], 0
    for r in range(B):
        lists.append(pages[at:at + n[r]].tolist())
        at += n[r]
    t = explicit_table(lists, ((lens - 1) % P) + 1, P, pool)
    nq = np.minimum(rng.integers(1, nq_max + 1, size=B), lens)
    t["qo_indptr"] = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    return t


@pytest.mark.parametrize("kv,nq_max,split", [("bf16", 1, False), ("bf16", 1, True),
                                               ("e4m3", 1, True), ("bf16", 4, True)])
def test_graph_captured_once_serves_later_plans(kv, nq_max, split):
    rng = np.random.default_rng(11 + nq_max)
    P, Hq, Hkv, D, pool = 16, 16, 4, 128, 400
    tabs = [_tables(rng, pool, P, B, 700, nq_max) for B in (7, 12, 3)]
    max_rows = max(int(t["qo_indptr"][-1]) for t in tabs)
    max_idx = max(len(t["indices"]) for t in tabs)
    # one KV pool for every plan; q rows drawn per plan
    w0 = custom_workload(1, Hq, Hkv, D, P, kv, "bf16", [1], pool_pages=pool)
    base = host_case(w0, 5, poison=False, table=explicit_table([[0]], [1], P, pool))
    kvd = to_device(base)
    q_buf = torch.zeros((max_rows, Hq, D), dtype=torch.bfloat16, device=DEV)
    out_buf = torch.zeros((max_rows, Hq, D), dtype=torch.float32, device=DEV)
    lse_buf = torch.zeros((max_rows, Hq), dtype=torch.float32, device=DEV)
    idx_buf = torch.zeros(max_idx, dtype=torch.int32, device=DEV)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    kw = dict(slots=256, balance=1, min_chunk_pages=1) if split else {}
    qrng = np.random.default_rng(99)
    graph, prev = None, None
    for step, t in enumerate(tabs):
        rows = int(t["qo_indptr"][-1])
        q32 = qrng.standard_normal((rows, Hq, D)).astype(np.float32)
        q = torch.from_numpy(q32).to(torch.bfloat16)
        qbits = q.view(torch.int16).numpy().view(np.uint16)
        q_buf[:rows].copy_(q.to(DEV))
        idx_buf[: len(t["indices"])].copy_(torch.from_numpy(t["indices"]))
        wr.plan(t["indptr"], idx_buf, t["last_page_len"], Hq, Hkv, D, P,
                q_data_type=torch.bfloat16,
                kv_data_type="e4m3" if kv == "e4m3" else torch.bfloat16,
                out_data_type=torch.float32, sm_scale=D ** -0.5, qo_indptr=t["qo_indptr"],
                capacity=CAP, **kw)
        info = wr.plan_info
        _say(kv, nq_max, split, "step", step, "rows", rows, "items", info["num_items"],
             "tasks", info["num_merge_tasks"])
        if split and step == 0:
            assert info["num_merge_tasks"] > 0  # the captured launch includes the merge
        args = dict(out=out_buf[:rows], lse=lse_buf[:rows], k_scale=kvd["k_scale"],
                    v_scale=kvd["v_scale"])
        if graph is None:
            wr.run(q_buf[:rows], kvd["kv"], **args)  # eager once: code objects loaded
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                wr.run(q_buf[:rows], kvd["kv"], **args)
        ref_out, ref_lse = attention.decode(qbits, base["kv"], t["indptr"], t["indices"],
                                            t["last_page_len"], num_kv_heads=Hkv,
                                            q_dtype="bf16", kv_dtype=kv, sm_scale=D ** -0.5,
                                            k_scale=base["k_scale"], v_scale=base["v_scale"],
                                            qo_indptr=t["qo_indptr"])
        for rep in range(3):
            out_buf.fill_(float("nan"))
            lse_buf.fill_(float("nan"))
            scratch = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            compare(out_buf[:rows], lse_buf[:rows], ref_out, ref_lse, kv)
            if rep == 0:
                first = out_buf[:rows].clone()
            else:
                assert torch.equal(out_buf[:rows], first)
            del scratch
    wr.close()


def test_fixed_capacity_plan_merges_a_prior_result():
    """run(prior=...) on a fixed-capacity plan (grids from the capacities,
    merge kernel always launched) gives the exact plan's bits, whole and
    split, and the oracle's merge of the two results."""
    from oracle import merge
    lens = [1, 17, 300, 64, 1000]
    w = custom_workload(5, 16, 4, 128, 16, "bf16", "bf16", lens, pool_pages=120)
    case = host_case(w, 5, poison=True)
    dc = to_device(case)
    ref_out, ref_lse = attention.decode_case(case)
    rng = np.random.default_rng(6)
    pv = rng.standard_normal(ref_out.shape).astype(np.float32)
    ps = (rng.standard_normal(ref_lse.shape) * 2 + 6).astype(np.float32)
    ps[0, :5] = -np.inf
    want_v, want_s = merge.merge_normalized(ref_out, ref_lse, pv.astype(np.float64),
                                            ps.astype(np.float64))
    prior = (torch.from_numpy(pv).to(DEV), torch.from_numpy(ps).to(DEV))
    for kw in (dict(min_chunk_pages=64), dict(slots=16, balance=1, min_chunk_pages=1)):
        res = []
        for cap in (None, dict(CAP, qo_len=1)):
            wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
            wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 16, 4, 128, 16,
                    q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16,
                    out_data_type=torch.float32, sm_scale=w.scale(), capacity=cap, **kw)
            out = torch.empty(dc["q"].shape, dtype=torch.float32, device=DEV)
            lse = torch.empty(dc["q"].shape[:2], dtype=torch.float32, device=DEV)
            for st in (pk._lib.STAGE_DECODE, pk._lib.STAGE_MERGE):
                wr.run(dc["q"], dc["kv"], out=out, lse=lse, stages=st, prior=prior)
            torch.cuda.synchronize()
            wr.close()
            compare(out, lse, want_v, want_s, "bf16")
            res.append((out, lse))
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_graph_replays_a_persistent_launch(kv):
    """A fixed-capacity plan with more work units (item x KV-head pair) than
    the device holds resident workgroups runs as a persistent launch, whose
    workgroups take units from counters in the workspace that the last one
    resets. Captured once, its replays (eager work between them) match the
    oracle and each other bit for bit, also for a second plan uploaded to the
    same workspace afterwards."""
    rng = np.random.default_rng(31 if kv == "bf16" else 32)
    P, Hq, Hkv, D, B, pool = 16, 32, 8, 128, 320, 8200
    tabs = [_tables(rng, pool, P, B, 400, 1) for _ in range(2)]
    cap = dict(items=1024, merge_tasks=512, partials=1024, qo_len=1)
    w0 = custom_workload(1, Hq, Hkv, D, P, kv, "bf16", [1], pool_pages=pool)
    base = host_case(w0, 7, poison=False, table=explicit_table([[0]], [1], P, pool))
    kvd = to_device(base)
    q_buf = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    out_buf = torch.zeros((B, Hq, D), dtype=torch.float32, device=DEV)
    lse_buf = torch.zeros((B, Hq), dtype=torch.float32, device=DEV)
    idx_buf = torch.zeros(max(len(t["indices"]) for t in tabs), dtype=torch.int32, device=DEV)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    qrng = np.random.default_rng(98)
    graph = None
    for step, t in enumerate(tabs):
        q = torch.from_numpy(qrng.standard_normal((B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
        qbits = q.view(torch.int16).numpy().view(np.uint16)
        q_buf.copy_(q.to(DEV))
        idx_buf.zero_()
        idx_buf[: len(t["indices"])].copy_(torch.from_numpy(t["indices"]))
        wr.plan(t["indptr"], idx_buf, t["last_page_len"], Hq, Hkv, D, P,
                q_data_type=torch.bfloat16,
                kv_data_type="e4m3" if kv == "e4m3" else torch.bfloat16,
                out_data_type=torch.float32, sm_scale=D ** -0.5, capacity=cap)
        info = wr.plan_info
        units = info["num_items"] * info["units_per_item"]
        _say("persistent", kv, "step", step, "items", info["num_items"], "units", units)
        assert units > 2 * cus  # more units than one workgroup per compute unit
        args = dict(out=out_buf, lse=lse_buf, k_scale=kvd["k_scale"], v_scale=kvd["v_scale"])
        if graph is None:
            wr.run(q_buf, kvd["kv"], **args)  # eager once: code objects loaded
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                wr.run(q_buf, kvd["kv"], **args)
        ref_out, ref_lse = attention.decode(qbits, base["kv"], t["indptr"], t["indices"],
                                            t["last_page_len"], num_kv_heads=Hkv,
                                            q_dtype="bf16", kv_dtype=kv, sm_scale=D ** -0.5,
                                            k_scale=base["k_scale"], v_scale=base["v_scale"])
        for rep in range(3):
            out_buf.fill_(float("nan"))
            lse_buf.fill_(float("nan"))
            scratch = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            compare(out_buf, lse_buf, ref_out, ref_lse, kv)
            if rep == 0:
                first = out_buf.clone()
            else:
                assert torch.equal(out_buf, first)
            del scratch
    wr.close()
