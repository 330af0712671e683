"""Cascade attention on the GPU: the merge_states kernel against the oracle's
normalised merge, non-causal q rows against the oracle, and the two-level
cascade against plain decode (oracle) over prefix + suffix pages."""
import math

import numpy as np
import pytest
import torch

import paged_kv_decode_plan_amd as pk
from gpu_helpers import TOL, compare, to_device, workspace
from oracle import attention, merge
from workloads import custom_workload, explicit_table, host_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print("[gpu-cascade]", *a, flush=True)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("in_dt,out_dt", [(torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16),
                                          (torch.bfloat16, torch.float32)])
def test_merge_states_matches_oracle(d, in_dt, out_dt):
    rng = np.random.default_rng(d)
    rows, heads = 37, 8
    va = torch.from_numpy(rng.standard_normal((rows, heads, d), dtype=np.float32)).to(in_dt)
    vb = torch.from_numpy(rng.standard_normal((rows, heads, d), dtype=np.float32)).to(in_dt)
    sa = (3 * rng.standard_normal((rows, heads))).astype(np.float32)
    sb = (3 * rng.standard_normal((rows, heads))).astype(np.float32)
    sa[0, :3] = -np.inf  # empty on one side
    sb[1, 2:5] = -np.inf
    _say("merge_states", d, in_dt, out_dt)
    v, s = pk.merge_state(va.to(DEV), torch.from_numpy(sa).to(DEV), vb.to(DEV),
                          torch.from_numpy(sb).to(DEV), out_dtype=out_dt)
    torch.cuda.synchronize()
    ref_v, ref_s = merge.merge_normalized(va.double().numpy(), sa, vb.double().numpy(), sb)
    got = v.double().cpu().numpy()
    bound = 1e-5 + (np.abs(ref_v) * 2.0 ** -8 if out_dt == torch.bfloat16 else 0.0)
    assert np.all(np.abs(got - ref_v) <= bound)
    np.testing.assert_allclose(s.cpu().numpy(), ref_s, rtol=0, atol=1e-5)


@pytest.mark.parametrize("d", [64, 96, 128, 192, 520])
@pytest.mark.parametrize("alias", ["a", "b"])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_merge_states_in_place(d, alias, dt):
    """Output written over one of the inputs (rows and LSEs): the same bits as
    the out-of-place merge, for head_dims whose (row, head) spans several
    wavefronts (96, 192, 520) as well as 64 and 128."""
    rng = np.random.default_rng(4000 + d)
    rows, heads = 53, 6
    va = torch.from_numpy(rng.standard_normal((rows, heads, d), dtype=np.float32)).to(dt).to(DEV)
    vb = torch.from_numpy(rng.standard_normal((rows, heads, d), dtype=np.float32)).to(dt).to(DEV)
    sa = torch.from_numpy((3 * rng.standard_normal((rows, heads))).astype(np.float32)).to(DEV)
    sb = torch.from_numpy((3 * rng.standard_normal((rows, heads))).astype(np.float32)).to(DEV)
    sa[0, :2] = -math.inf
    sb[3, 1:4] = -math.inf
    _say("merge_states in place", d, alias, dt)
    want_v, want_s = pk.merge_state(va, sa, vb, sb)
    torch.cuda.synchronize()
    if alias == "a":
        v, s = va.clone(), sa.clone()
        pk.merge_state(v, s, vb, sb, v_out=v, s_out=s)
    else:
        v, s = vb.clone(), sb.clone()
        pk.merge_state(va, sa, v, s, v_out=v, s_out=s)
    torch.cuda.synchronize()
    assert torch.equal(v, want_v)
    assert torch.equal(s, want_s)
    ref_v, ref_s = merge.merge_normalized(va.double().cpu().numpy(), sa.cpu().numpy(),
                                          vb.double().cpu().numpy(), sb.cpu().numpy())
    bound = 1e-5 + (np.abs(ref_v) * 2.0 ** -8 if dt == torch.bfloat16 else 0.0)
    assert np.all(np.abs(v.double().cpu().numpy() - ref_v) <= bound)
    np.testing.assert_allclose(s.cpu().numpy(), ref_s, rtol=0, atol=1e-5)


def test_merge_states_both_empty_is_empty():
    va = torch.ones((2, 1, 4), device=DEV)
    s = torch.full((2, 1), -math.inf, device=DEV)
    v, so = pk.merge_state(va, s, va, s)
    torch.cuda.synchronize()
    assert torch.all(v == 0) and torch.all(torch.isinf(so)) and torch.all(so < 0)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_non_causal_rows_more_than_tokens(kv):
    nq = [20, 3, 9]  # request 0 has 5 tokens and 20 query rows
    P = 16
    t = explicit_table([[3, 7][:1], [1, 9, 4], list(range(10, 29))], [5, 5, 12], P, 30)
    w = custom_workload(3, 16, 4, 128, P, kv, "bf16", t["kv_lens"].tolist(), pool_pages=30)
    case = host_case(w, 5, poison=True, table=t)
    qrows = np.random.default_rng(1).standard_normal((sum(nq), 16, 128)).astype(np.float32)
    qbits = torch.from_numpy(qrows).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    case["q"] = qbits
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    ref_out, ref_lse = attention.decode(case["q"], case["kv"], t["indptr"], t["indices"],
                                        t["last_page_len"], num_kv_heads=4, q_dtype="bf16",
                                        kv_dtype=kv, sm_scale=w.scale(), k_scale=case["k_scale"],
                                        v_scale=case["v_scale"], qo_indptr=qo, causal=False)
    dc = to_device(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
        wr.plan(t["indptr"], dc["indices"], t["last_page_len"], 16, 4, 128, P,
                q_data_type=torch.bfloat16, kv_data_type="e4m3" if kv == "e4m3" else torch.bfloat16,
                out_data_type=torch.float32, sm_scale=w.scale(), qo_indptr=qo, causal=False, **kw)
        out, lse = wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                          v_scale=dc["v_scale"])
        torch.cuda.synchronize()
        wr.close()
        compare(out, lse, ref_out, ref_lse, kv)


def _cascade_case(kv, g, seed):
    """Two prefix groups (40 and 7 full pages) over 8 requests with their own
    suffixes; the full page lists are prefix + suffix."""
    P, hkv = 16, 2
    rng = np.random.default_rng(seed)
    groups = [(40, [0, 1, 2, 3, 4]), (7, [5, 6, 7])]
    suffix_pages = rng.integers(1, 21, size=8)
    pool = sum(n for n, _ in groups) + int(suffix_pages.sum()) + 9
    perm = rng.permutation(pool).tolist()
    prefix_lists, at = [], 0
    for n, _ in groups:
        prefix_lists.append(perm[at:at + n])
        at += n
    suffix_lists = []
    for r in range(8):
        suffix_lists.append(perm[at:at + int(suffix_pages[r])])
        at += int(suffix_pages[r])
    last = rng.integers(1, P + 1, size=8).tolist()
    owner = [0] * 5 + [1] * 3
    full = explicit_table([prefix_lists[owner[r]] + suffix_lists[r] for r in range(8)], last, P,
                          pool)
    w = custom_workload(8, hkv * g, hkv, 128, P, kv, "bf16", full["kv_lens"].tolist(),
                        pool_pages=pool)
    case = host_case(w, seed, poison=True, table=full)
    shared = explicit_table(prefix_lists, [P, P], P, pool)
    unique = explicit_table(suffix_lists, last, P, pool)
    return w, case, shared, unique, np.array([0, 5, 8], np.int32)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_cascade_matches_decode_over_prefix_plus_suffix(kv, g, out_dt):
    w, case, shared, unique, groups = _cascade_case(kv, g, 20 + g)
    _say("cascade", kv, g, out_dt)
    ref_out, ref_lse = attention.decode_case(case)
    dc = to_device(case)
    cw = pk.CascadeBatchDecodeWrapper(workspace(), "NHD")
    cw.plan(shared["indptr"], torch.from_numpy(shared["indices"]).to(DEV), shared["last_page_len"],
            groups, unique["indptr"], torch.from_numpy(unique["indices"]).to(DEV),
            unique["last_page_len"], w.num_qo_heads, w.num_kv_heads, 128, 16,
            q_data_type=torch.bfloat16, kv_data_type="e4m3" if kv == "e4m3" else torch.bfloat16,
            out_data_type=out_dt, sm_scale=w.scale())
    out, lse = cw.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                      v_scale=dc["v_scale"])
    torch.cuda.synchronize()
    cw.close()
    assert out.dtype == out_dt
    compare(out, lse, ref_out, ref_lse, kv, out_dtype="bf16" if out_dt == torch.bfloat16 else "f32")


def test_full_size_cascade_sampled_requests():
    """The 64-request, 8192-token shared-prefix workload at full size in the
    bench's configuration; sampled requests against decode over their full
    page lists."""
    from gpu_helpers import sample_request_case
    from workloads import CONFIGS, device_case
    name = "cascade_prefix8k_bf16"
    w = CONFIGS[name]
    seed = list(CONFIGS).index(name) + 1
    _say("full-size", name, "seed", seed)
    dc = device_case(w, seed, DEV, poison=True)
    sh, un = dc["shared"], dc["unique"]
    cw = pk.CascadeBatchDecodeWrapper(workspace(), "NHD")
    cw.plan(sh["indptr"], torch.from_numpy(sh["indices"]).to(DEV), sh["last_page_len"],
            dc["group_qo_indptr"], un["indptr"], torch.from_numpy(un["indices"]).to(DEV),
            un["last_page_len"], w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
            q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16,
            out_data_type=torch.float32, sm_scale=w.scale())
    out, lse = cw.run(dc["q"], dc["kv"], return_lse=True)
    torch.cuda.synchronize()
    cw.close()
    assert torch.isfinite(out).all()
    for r in (0, 31, w.batch - 1):
        sub = sample_request_case(dc, r)
        ref_out, ref_lse = attention.decode_case(sub)
        compare(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, "bf16")
    del dc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["whole", "folded", "merge_kernel"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_run_merges_a_prior_result(mode, out_dtype):
    """run(prior=(v, lse)) writes the merge of its own result with another
    normalised result of the same rows (the cascade's other level), on the
    three paths that write final rows: an unsplit item's epilogue, the merge
    folded into the decode kernel, and the merge kernel. Rows whose prior is
    empty (LSE -inf) keep the run's own result."""
    lens = [300, 17, 90, 1]
    w = custom_workload(len(lens), 16, 4, 128, 16, "bf16", "bf16", lens, pool_pages=40)
    case = host_case(w, 333, poison=True)
    ref_v, ref_s = attention.decode_case(case)
    rng = np.random.default_rng(334)
    pv = rng.standard_normal(ref_v.shape).astype(np.float32)
    ps = (rng.standard_normal(ref_s.shape) * 3 + 5).astype(np.float32)
    ps[1, :] = -np.inf  # an empty prior for every head of request 1
    ps[2, 3] = -np.inf
    want_v, want_s = merge.merge_normalized(ref_v, ref_s, pv.astype(np.float64), ps.astype(np.float64))
    dc = to_device(case)
    kw = {"whole": dict(min_chunk_pages=64), "folded": dict(slots=64, balance=1, min_chunk_pages=5),
          "merge_kernel": dict(slots=64, balance=1, min_chunk_pages=1)}[mode]
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    odt = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 16, 4, 128, 16,
            q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16, out_data_type=odt, **kw)
    info = wr.plan_info
    if mode == "whole":
        assert info["num_split_requests"] == 0
    else:
        assert info["num_split_requests"] > 0 and info["merge_folded"] == (mode == "folded")
    out, lse = wr.run(dc["q"], dc["kv"], return_lse=True,
                      prior=(torch.from_numpy(pv).cuda(), torch.from_numpy(ps).cuda()))
    torch.cuda.synchronize()
    wr.close()
    compare(out, lse, want_v, want_s, "bf16", out_dtype=out_dtype)
