"""HIP path (through the C ABI) against the float64 oracle on the same seeded inputs.

Tolerances: max-abs 2e-3 for fp32/bf16 KV and 3e-2 for e4m3 KV (against the
same dequantised values), compared in fp32 output before rounding; bf16
output adds half an ulp of rounding. Index-exact properties (the gather
probe, page-permutation invariance, determinism, single key) are bit-exact.
"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import (compare, oracle_for, out_to_f64, run_hip, sample_request_case,
                         to_device)
from workloads import CONFIGS, custom_workload, device_case, host_case, read_mask

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu]", *a, flush=True)


# ------------------------------------------------------------------ small cases, every kernel

SMALL = []
for kv in ("f32", "bf16", "e4m3"):
    for d in (64, 128):
        for g in (1, 2, 4, 8, 16):
            if g == 16 and (kv == "f32" or d == 64):
                continue  # group 16 exists only on the MFMA path
            SMALL.append((kv, d, g, "f32" if kv == "f32" else "bf16"))
# fp32 queries over bf16 / e4m3 KV take the vector-ALU kernel
SMALL += [("bf16", 128, 4, "f32"), ("e4m3", 128, 8, "f32"), ("bf16", 128, 1, "f32")]


@pytest.mark.parametrize("kv,d,g,qd", SMALL)
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_small_ragged_matches_oracle(kv, d, g, qd, split):
    hkv = 2
    lens = [1, 15, 16, 17, 100, 333, 700, 64, 3]
    P = 16
    w = custom_workload(len(lens), hkv * g, hkv, d, P, kv, qd, lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 7)
    seed = 100 + 7 * d + g
    case = host_case(w, seed, poison=True)
    _say("small", kv, d, g, qd, split, "seed", seed)
    ref_out, ref_lse = oracle_for(case)
    dc = to_device(case)
    kw = dict(slots=4, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(dc, **kw)
    if split == "forced":
        assert info["num_split_requests"] > 0
    compare(out, lse, ref_out, ref_lse, kv)


@pytest.mark.parametrize("kv,qd", [("bf16", "bf16"), ("e4m3", "bf16"), ("f16", "f16")])
@pytest.mark.parametrize("hkv", [3, 4, 8, 16])
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_one_or_two_kv_heads_per_workgroup(kv, qd, hkv, split):
    """An odd KV head count keeps one KV head per workgroup; an even one may
    take pairs (per form): both against the oracle."""
    lens = [1, 15, 16, 17, 100, 333, 700, 64, 3]
    w = custom_workload(len(lens), 4 * hkv, hkv, 128, 16, kv, qd, lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 5)
    case = host_case(w, 300 + hkv, poison=True)
    _say("kv heads", kv, hkv, split)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=8, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(to_device(case), **kw)
    assert info["units_per_item"] in (hkv, hkv // 2, hkv // 8)
    compare(out, lse, ref_out, ref_lse, kv)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("P", [1, 2, 4, 8, 16, 32, 64, 128])
def test_page_sizes(P, kv):
    lens = [1, P, P + 1, 3 * P + 5, 257]
    w = custom_workload(len(lens), 8, 2, 128, P, kv, "bf16", lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 3)
    case = host_case(w, 40 + P, poison=True)
    _say("page size", P, kv)
    ref_out, ref_lse = oracle_for(case)
    dc = to_device(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(dc, **kw)
        compare(out, lse, ref_out, ref_lse, kv)


@pytest.mark.parametrize("kv,qd,d", [("f32", "f32", 64), ("bf16", "bf16", 128), ("e4m3", "bf16", 128),
                                      ("f16", "f16", 128), ("e2m1", "bf16", 128), ("i4", "bf16", 128)])
@pytest.mark.parametrize("P", [256, 1024])
def test_large_pages(P, kv, qd, d):
    """Pages up to the largest size plan() accepts (1024 tokens), on every
    kernel form: lengths inside one page, at page ends and across several."""
    lens = [1, P - 1, P, P + 3, 2 * P + 17]
    w = custom_workload(len(lens), 8, 2, d, P, kv, qd, lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 2)
    case = host_case(w, 70 + P, poison=True)
    _say("large pages", P, kv, qd, d)
    ref_out, ref_lse = oracle_for(case)
    dc = to_device(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(dc, **kw)
        compare(out, lse, ref_out, ref_lse, kv)


@pytest.mark.parametrize("kv", ["f32", "bf16", "e4m3"])
def test_bf16_output_rounding(kv):
    lens = [5, 200, 31]
    w = custom_workload(3, 8, 2, 128, 16, kv, "bf16", lens, pool_pages=20)
    case = host_case(w, 9, poison=True)
    ref_out, ref_lse = oracle_for(case)
    out, lse, _ = run_hip(to_device(case), out_dtype="bf16")
    assert out.dtype == torch.bfloat16
    compare(out, lse, ref_out, ref_lse, kv, out_dtype="bf16")


def test_single_seq_fp32_config_full():
    """single_seq_fp32: B=1, 4/4 heads, D=64, P=16, 512 tokens in a 64-page pool."""
    w = CONFIGS["single_seq_fp32"]
    case = host_case(w, 1, poison=True)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=64, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "f32")


# ------------------------------------------------------------------ exact properties

def _encode(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if kv_dtype == "f32":
        return t.numpy()
    if kv_dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _probe_case(kv_dtype, lens, P, hq, hkv, d, seed, q_dtype="f32"):
    """V carries the page id in base-16 digits and the slot, all small integers
    that every KV format stores exactly; one token per request gets a logit 200
    above all others, so every other weight is exactly 0 in fp32."""
    w = custom_workload(len(lens), hq, hkv, d, P, kv_dtype, q_dtype, lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 5)
    case = host_case(w, seed, poison=True)
    rng = np.random.default_rng(seed)
    npg = case["num_pages"]
    vals = np.zeros((npg, 2, P, hkv, d), np.float32)
    pages = np.arange(npg)
    vals[:, 1, :, :, 0] = (pages // 256)[:, None, None]
    vals[:, 1, :, :, 1] = ((pages // 16) % 16)[:, None, None]
    vals[:, 1, :, :, 2] = (pages % 16)[:, None, None]
    vals[:, 1, :, :, 3] = np.arange(P)[None, :, None] % 16
    vals[:, 1, :, :, 4] = np.arange(P)[None, :, None] // 16
    kscale = 1.0
    if kv_dtype == "e4m3":
        big = 448.0
        kscale = 200.0 * np.sqrt(d) / big
        case["k_scale"] = np.full_like(case["k_scale"], kscale)
        case["v_scale"] = np.ones_like(case["v_scale"])
    else:
        big = 200.0 * np.sqrt(d)
    targets = []
    for r in range(len(lens)):
        t = int(rng.integers(0, lens[r]))
        page = int(case["indices"][case["indptr"][r] + t // P])
        vals[page, 0, t % P, :, 0] = big
        targets.append((page, t % P))
    unread = ~read_mask(case, P)
    enc = _encode(vals, kv_dtype)
    nan = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}[kv_dtype]
    enc[:, 0][unread] = nan
    enc[:, 1][unread] = nan
    case["kv"] = enc
    qv = np.zeros((len(lens), hq, d), np.float32)
    qv[:, :, 0] = 1.0
    case["q"] = qv if q_dtype == "f32" else _encode(qv, "bf16")
    return case, targets


@pytest.mark.parametrize("kv,d,qd", [("f32", 64, "f32"), ("bf16", 128, "bf16"),
                                     ("e4m3", 128, "bf16"), ("bf16", 64, "bf16")])
@pytest.mark.parametrize("forced_split", [False, True])
def test_gather_index_probe_bit_exact(kv, d, qd, forced_split):
    """One dominant token per request: out must equal that token's V exactly,
    which reads back (page id, slot) — the gather mapping, bit for bit."""
    lens = [1, 2, 17, 48, 255, 1000, 4096, 33]
    P, hq, hkv = 16, 8, 4
    case, targets = _probe_case(kv, lens, P, hq, hkv, d, 77, qd)
    kw = dict(slots=16, balance=1, min_chunk_pages=1) if forced_split else {}
    out, _, info = run_hip(to_device(case), **kw)
    o = out.cpu().numpy()
    for r, (page, slot) in enumerate(targets):
        got_page = o[r, :, 0] * 256 + o[r, :, 1] * 16 + o[r, :, 2]
        got_slot = o[r, :, 3] + 16 * o[r, :, 4]
        assert np.all(got_page == page) and np.all(got_slot == slot), (r, page, slot, o[r, 0, :5])
        assert np.all(o[r, :, 5:] == 0)


def test_page_permutation_invariance_bit_exact():
    lens = [100, 37, 512, 9]
    w = custom_workload(4, 16, 4, 128, 16, "bf16", "bf16", lens, pool_pages=60)
    case = host_case(w, 3, poison=True)
    out1, lse1, _ = run_hip(to_device(case))
    perm = np.random.default_rng(5).permutation(case["num_pages"])
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    case2 = dict(case)
    case2["kv"] = case["kv"][inv]
    case2["indices"] = perm[case["indices"]].astype(np.int32)
    out2, lse2, _ = run_hip(to_device(case2))
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_run_to_run_determinism():
    w = custom_workload(6, 32, 8, 128, 16, "bf16", "bf16", [3000, 20, 700, 1, 4096, 65], pool_pages=700)
    case = host_case(w, 12, poison=True)
    dc = to_device(case)
    a = run_hip(dc, slots=32, balance=1, min_chunk_pages=1)
    b = run_hip(dc, slots=32, balance=1, min_chunk_pages=1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_single_key_returns_v_exactly():
    w = custom_workload(3, 8, 2, 128, 16, "bf16", "bf16", [1, 1, 1], pool_pages=5)
    case = host_case(w, 2, poison=True)
    out, lse, _ = run_hip(to_device(case))
    ref, _ = oracle_for(case)
    assert np.array_equal(out_to_f64(out), ref)


def test_constant_v_returns_v():
    w = custom_workload(3, 8, 2, 128, 16, "f32", "f32", [700, 1, 40], pool_pages=50)
    case = host_case(w, 4, poison=True)
    c = np.linspace(-3, 3, 128).astype(np.float32)
    finite = ~np.isnan(case["kv"][:, 1])
    case["kv"][:, 1] = np.where(finite, c, np.nan)
    out, _, _ = run_hip(to_device(case), slots=8, balance=1, min_chunk_pages=1)
    np.testing.assert_allclose(out.cpu().numpy(), np.broadcast_to(c, out.shape), rtol=1e-5, atol=1e-6)


def test_split_equals_unsplit_within_tolerance():
    w = custom_workload(4, 16, 4, 128, 16, "bf16", "bf16", [5000, 300, 64, 1234], pool_pages=500)
    case = host_case(w, 8, poison=True)
    dc = to_device(case)
    a, la, ia = run_hip(dc, slots=1, balance=1, min_chunk_pages=1000)
    b, lb, ib = run_hip(dc, slots=64, balance=1, min_chunk_pages=1)
    assert ia["num_partials"] == 0 and ib["num_partials"] > 0
    assert float((a - b).abs().max()) < 1e-4
    assert float((la - lb).abs().max()) < 1e-4


def test_shared_prefix_pages_are_legal():
    """The pages' worked example: two requests share their first three pages."""
    from workloads import explicit_table
    lists = [[7, 2, 15, 88, 3], [7, 2, 15, 41]]
    table = explicit_table(lists, [16, 9], 16, num_pages=90)
    w = custom_workload(2, 8, 2, 128, 16, "bf16", "bf16", [int(x) for x in table["kv_lens"]],
                        pool_pages=90)
    case = host_case(w, 6, poison=True, table=table)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "bf16")


# ------------------------------------------------------------------ full-size workloads

FULL = ["llama3_8b_bf16", "ragged_loguniform_bf16", "long_ctx_gqa8_bf16", "fp8_kv_e4m3"]


def _run_full(dc, **plan_kw):
    """run() of a full-size device case (default plan unless plan_kw), with the
    plan's split requests."""
    import paged_kv_decode_plan_amd as pk
    from gpu_helpers import workspace
    w = dc["workload"]
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], w.num_qo_heads, w.num_kv_heads,
            w.head_dim, w.page_size, q_data_type=dc["q"].dtype,
            kv_data_type=w.kv_dtype if w.kv_dtype == "e4m3" else dc["kv"].dtype,
            out_data_type=torch.float32, sm_scale=w.scale(), **plan_kw)
    out, lse = wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                      v_scale=dc["v_scale"])
    torch.cuda.synchronize()
    info = wr.plan_info
    split = wr._plan.worklist()[2].tolist()
    wr.close()
    return out, lse, info, split


def _check_requests(dc, out, lse, rows, kv):
    for n, r in enumerate(rows):
        sub = sample_request_case(dc, r)
        ref_out, ref_lse = oracle_for(sub)
        if n % 8 == 0:
            _say(f"  request {r} ({n + 1}/{len(rows)}), {int(dc['kv_lens'][r])} tokens")
        compare(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, kv)


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """Full-size batch in the bench's launch configuration (the device-default
    plan), compared element by element with the oracle: every request of the
    Llama-shaped batch and of the long-context pair; every split request of
    the ragged batch and 16 more; 24 requests of the fp8 batch (whose default
    plan splits none), then every split request of a plan that splits (balance
    4) over the same device data."""
    w = CONFIGS[name]
    seed = list(CONFIGS).index(name) + 1
    _say("full-size", name, "seed", seed)
    dc = device_case(w, seed, "cuda:0", poison=True)
    out, lse, info, split = _run_full(dc)
    _say("plan", info)
    assert np.all(np.isfinite(out_to_f64(out)))
    lens = dc["kv_lens"]
    rng = np.random.default_rng(seed)
    if name in ("llama3_8b_bf16", "long_ctx_gqa8_bf16"):
        rows = list(range(w.batch))
    else:
        others = [r for r in range(w.batch) if r not in set(split)]
        extra = 16 if name == "ragged_loguniform_bf16" else 24
        rows = sorted(set(split) | {int(np.argmin(lens)), int(np.argmax(lens))}
                      | set(rng.choice(others, size=extra, replace=False).tolist()))
    if name == "ragged_loguniform_bf16":
        assert len(split) > 0
    _check_requests(dc, out, lse, rows, w.kv_dtype)
    if name == "fp8_kv_e4m3":
        out2, lse2, info2, split2 = _run_full(dc, balance=4)
        _say("balance 4 plan", info2)
        assert len(split2) > 0
        _check_requests(dc, out2, lse2, split2, w.kv_dtype)
    del dc
    torch.cuda.empty_cache()


# Decode workgroups per compute unit that the library keeps by default for a
# one-token plan on the MFMA kernel (an LDS reservation): one for 16-bit and
# e4m3 KV, two for e2m1, three for int4.
DEFAULT_RESIDENCY = {"bf16": 1, "f16": 1, "e4m3": 1, "e2m1": 2, "i4": 3}


@pytest.mark.parametrize("name", [n for n in CONFIGS if CONFIGS[n].shared_prefix is None])
def test_device_default_plan_matches_the_oracle_rule(name):
    """The plan run() uses by default (slots = 0: the device's compute units
    times the kernel's resident workgroups) against the oracle's rule with the
    same slots, slots per compute unit, balance and shortest chunk, bit for
    bit; the slot count is the compute units times that residency."""
    import paged_kv_decode_plan_amd as pk
    from oracle import plan as oplan
    from workloads import page_table
    w = CONFIGS[name]
    t = page_table(w, seed=list(CONFIGS).index(name) + 1)
    info, items, merge, split = pk.plan_partition(
        t["indptr"], t["last_page_len"], w.num_qo_heads, w.num_kv_heads, w.head_dim,
        w.page_size, kv_dtype=w.kv_dtype, q_dtype=w.q_dtype, slots=0,
        qo_indptr=t["qo_indptr"], kv_scale=w.kv_scale)
    _say("default plan", name, {k: info[k] for k in ("slots", "slots_per_cu", "num_items",
                                                     "num_partials", "units_per_item")})
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert info["slots"] == info["slots_per_cu"] * cus
    one_token = t["qo_indptr"] is None and w.head_dim == 128 and w.q_dtype != "f32"
    if one_token and w.kv_dtype in DEFAULT_RESIDENCY:
        assert info["slots_per_cu"] == DEFAULT_RESIDENCY[w.kv_dtype]
    ref = oplan.plan(t["indptr"], t["last_page_len"], w.page_size, info["units_per_item"],
                     info["slots"], info["balance"], info["min_chunk_pages"], t["qo_indptr"],
                     info["queries_per_item"], slots_per_cu=info["slots_per_cu"])
    assert info["chunk_pages"] == ref["chunk_pages"]
    assert np.array_equal(items, ref["items"])
    assert np.array_equal(merge, ref["merge_indptr"])
    assert np.array_equal(split, ref["split_requests"])


# ------------------------------------------------------------------ merge paths

def _merge_case(lens, seed, kv="bf16"):
    w = custom_workload(len(lens), 16, 4, 128, 16, kv, "bf16", lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 4)
    return w, host_case(w, seed, poison=True)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("chunks", [8, 16, 17])
def test_fold_takes_up_to_sixteen_chunks(kv, chunks):
    """One request cut into exactly `chunks` chunks of four pages (a pair of
    KV heads per workgroup, so at most 34 split workgroups): up to sixteen
    chunks the merge is folded into the decode kernel, seventeen take the
    merge kernel; either way the rows match the oracle, and a second run
    (fold counters back at zero) gives the same bits."""
    import paged_kv_decode_plan_amd as pk
    from gpu_helpers import workspace
    lens = [64 * chunks - 5, 40, 64, 3]
    w, case = _merge_case(lens, 40 + chunks, kv)
    ref_out, ref_lse = oracle_for(case)
    dc = to_device(case)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 16, 4, 128, 16,
            q_data_type=torch.bfloat16, kv_data_type="e4m3" if kv == "e4m3" else torch.bfloat16,
            out_data_type=torch.float32, sm_scale=w.scale(), slots=1024, balance=1,
            min_chunk_pages=4)
    info = wr.plan_info
    _say("fold limit", kv, chunks, {k: info[k] for k in ("num_items", "num_split_requests",
                                                          "merge_folded", "chunk_pages")})
    assert info["chunk_pages"] == 4 and info["num_split_requests"] == 1
    assert info["merge_folded"] == (1 if chunks <= 16 else 0)
    outs = []
    for _ in range(2):
        out, lse = wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                          v_scale=dc["v_scale"])
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, kv)
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    wr.close()


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_folded_merge_matches_oracle_and_resets(kv):
    """Short splits (at most sixteen chunks per request, few workgroups):
    run() folds the merge into the decode kernel; the result matches the
    oracle and repeating the run (arrival counters back at zero) gives the
    same bits."""
    import paged_kv_decode_plan_amd as pk
    from gpu_helpers import workspace
    w, case = _merge_case([300, 64, 900, 17], 31, kv)
    ref_out, ref_lse = oracle_for(case)
    dc = to_device(case)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 16, 4, 128, 16,
            q_data_type=torch.bfloat16, kv_data_type="e4m3" if kv == "e4m3" else torch.bfloat16,
            out_data_type=torch.float32, sm_scale=w.scale(), slots=32, balance=1,
            min_chunk_pages=16)
    info = wr.plan_info
    assert info["num_split_requests"] > 0 and info["merge_folded"] == 1
    outs = []
    for _ in range(3):
        out, lse = wr.run(dc["q"], dc["kv"], return_lse=True, k_scale=dc["k_scale"],
                          v_scale=dc["v_scale"])
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, kv)
        outs.append((out.clone(), lse.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    # the stages kept apart (decode writes partial states, the merge kernel folds)
    o2, l2 = torch.empty_like(outs[0][0]), torch.empty_like(outs[0][1])
    for st in (pk._lib.STAGE_DECODE, pk._lib.STAGE_MERGE):
        wr.run(dc["q"], dc["kv"], out=o2, lse=l2, k_scale=dc["k_scale"], v_scale=dc["v_scale"],
               stages=st)
    torch.cuda.synchronize()
    compare(o2, l2, ref_out, ref_lse, kv)
    wr.close()


def test_long_splits_use_the_merge_kernel():
    w, case = _merge_case([3000, 64, 2000], 32)
    ref_out, ref_lse = oracle_for(case)
    out, lse, info = run_hip(to_device(case), slots=256, balance=1, min_chunk_pages=1)
    assert info["num_split_requests"] > 0 and info["merge_folded"] == 0
    compare(out, lse, ref_out, ref_lse, "bf16")


def test_page_id_check_rejects_ids_outside_the_pool():
    """pkd_check_page_ids counts ids outside the pool; run(check_page_ids=True)
    raises on such a table before launching anything and runs normally on a
    valid one."""
    import paged_kv_decode_plan_amd as pk
    from paged_kv_decode_plan_amd import _lib
    lens = [40, 17, 100]
    w = custom_workload(3, 8, 2, 128, 16, "bf16", "bf16", lens, pool_pages=20)
    case = host_case(w, 61, poison=True)
    dc = to_device(case)
    num_pages = int(dc["kv"].shape[0])
    ref_out, ref_lse = oracle_for(case)
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(torch.empty(1 << 20, dtype=torch.uint8,
                                                           device="cuda:0"), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 8, 2, 128, 16,
            q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16,
            out_data_type=torch.float32)
    out, lse = wr.run(dc["q"], dc["kv"], return_lse=True, check_page_ids=True)
    torch.cuda.synchronize()
    compare(out, lse, ref_out, ref_lse, "bf16")
    for pos, bad_id in [(3, num_pages), (int(dc["indices"].numel()) - 1, -1)]:
        bad = dc["indices"].clone()
        bad[pos] = bad_id
        cnt, first = ctypes.c_int64(), ctypes.c_int64()
        _lib.check(_lib.load().pkd_check_page_ids(
            ctypes.c_void_p(bad.data_ptr()), ctypes.c_int64(bad.numel()), ctypes.c_int32(num_pages),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(cnt),
            ctypes.byref(first)))
        assert (cnt.value, first.value) == (1, pos)
        wr.plan(dc["indptr"], bad, dc["last_page_len"], 8, 2, 128, 16,
                q_data_type=torch.bfloat16, kv_data_type=torch.bfloat16,
                out_data_type=torch.float32)
        with pytest.raises(_lib.PkdError, match="outside the pool"):
            wr.run(dc["q"], dc["kv"], check_page_ids=True)
    wr.close()


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "e2m1"])
def test_separate_k_and_v_pools(kv):
    """A (k, v) pair of pools gives the combined pool's result bit for bit:
    as views into the combined tensor, as separate contiguous tensors, and
    as pools whose pages are padded (page stride larger than the page)."""
    lens = [1, 37, 300, 64, 129]
    w = custom_workload(len(lens), 16, 4, 128, 16, kv, "bf16", lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 4)
    case = host_case(w, 520, poison=True)
    _say("separate pools", kv)
    dc = to_device(case)
    out0, lse0, _ = run_hip(dc)
    k, v = dc["kv"][:, 0], dc["kv"][:, 1]
    padded = torch.zeros((k.shape[0], k.shape[1] + 3) + tuple(k.shape[2:]), dtype=k.dtype,
                         device=k.device)
    kp, vp = padded.clone(), padded.clone()
    kp[:, :k.shape[1]] = k
    vp[:, :v.shape[1]] = v
    for pools in [(k, v), (k.contiguous(), v.contiguous()),
                  (kp[:, :k.shape[1]], vp[:, :v.shape[1]])]:
        out, lse, _ = run_hip(dc, kv=pools)
        assert torch.equal(out, out0) and torch.equal(lse, lse0)


def test_large_batch_of_short_requests():
    """Two thousand requests of 1-400 tokens: a plan of thousands of work
    items and a grid of thousands of workgroups, checked on sampled requests
    against the oracle."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 401, 2048)]
    w = custom_workload(len(lens), 8, 2, 128, 16, "bf16", "bf16", lens)
    _say("large batch", len(lens), "requests", sum(lens), "tokens")
    dc = device_case(w, 78, "cuda:0", poison=True)
    out, lse, info = run_hip(dc)
    _say("plan", info)
    assert info["num_items"] >= len(lens)
    o = out_to_f64(out)
    assert np.all(np.isfinite(o))
    for r in sorted({0, 1, 1023, 2047, int(np.argmax(lens)), int(np.argmin(lens))}):
        sub = sample_request_case(dc, r)
        ref_out, ref_lse = oracle_for(sub)
        compare(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, "bf16")


def test_two_streams_two_workspaces():
    """Two plans with their own workspaces, planned and run on two streams
    (default priority) with their launches interleaved, give the results of
    the same runs made one after the other, bit for bit, and match the
    oracle."""
    import paged_kv_decode_plan_amd as pk
    cases = []
    for seed, (kv, lens) in enumerate([("bf16", [900, 33, 1, 2500]), ("e4m3", [64, 1700, 400])]):
        w = custom_workload(len(lens), 16, 4, 128, 16, kv, "bf16", lens,
                            pool_pages=sum(-(-x // 16) for x in lens) + 3)
        cases.append(host_case(w, 880 + seed, poison=True))
    seq = [run_hip(to_device(c), slots=32, balance=1, min_chunk_pages=1)[:2] for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wrappers, dcs = [], []
    for c, st in zip(cases, streams):
        dc = to_device(c)
        wr = pk.BatchDecodeWithPagedKVCacheWrapper(
            torch.empty(16 << 20, dtype=torch.uint8, device="cuda:0"), "NHD")
        w = dc["workload"]
        with torch.cuda.stream(st):
            wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], 16, 4, 128, 16,
                    q_data_type=torch.bfloat16,
                    kv_data_type=w.kv_dtype if w.kv_dtype == "e4m3" else torch.bfloat16,
                    out_data_type=torch.float32, slots=32, balance=1, min_chunk_pages=1)
        wrappers.append(wr)
        dcs.append(dc)
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):  # interleaved launches on the two streams
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
    for c, (o, l) in zip(cases, seq):
        ref_out, ref_lse = oracle_for(c)
        compare(o, l, ref_out, ref_lse, c["workload"].kv_dtype)
    for wr in wrappers:
        wr.close()
