"""Row-wise (per-token) e4m3 scales on the GPU against the oracle.

One fp32 scale per (token, KV head) for K and for V ([num_pages, Hkv,
page_size]); same 3e-2 max-abs tolerance as per-page e4m3 against the same
dequantised values.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import compare, oracle_for, out_to_f64, run_hip, sample_request_case, to_device
from workloads import CONFIGS, custom_workload, device_case, host_case

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 100, 333, 700, 64, 3]


def _say(*a):
    print("[gpu-rowwise]", *a, flush=True)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_small_ragged_rowwise(g, split):
    w = custom_workload(len(LENS), 2 * g, 2, 128, 16, "e4m3", "bf16", LENS,
                        pool_pages=sum(-(-x // 16) for x in LENS) + 7, kv_scale="token")
    case = host_case(w, 500 + g, poison=True)
    _say("small", g, split)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=64, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(to_device(case), **kw)
    if split == "forced":
        assert info["num_split_requests"] > 0
    compare(out, lse, ref_out, ref_lse, "e4m3")


@pytest.mark.parametrize("P", [1, 2, 4, 16, 32, 64])
def test_rowwise_page_sizes(P):
    lens = [1, P, P + 1, 3 * P + 5, 257]
    w = custom_workload(len(lens), 8, 2, 128, P, "e4m3", "bf16", lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 3, kv_scale="token")
    case = host_case(w, 60 + P, poison=True)
    _say("pages", P)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "e4m3")


def test_rowwise_with_several_new_tokens():
    lens, nq = [40, 333, 17, 100], [30, 7, 4, 16]
    w = custom_workload(4, 16, 4, 128, 16, "e4m3", "bf16", lens, pool_pages=40,
                        qo_lens=nq, kv_scale="token")
    case = host_case(w, 77, poison=True)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=64, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "e4m3")


def test_rowwise_scales_equal_to_page_scales_match_page_path():
    """Row-wise scales repeating each page's scale give the per-page result
    (within rounding: the scale enters the score at a different point)."""
    w = custom_workload(len(LENS), 16, 2, 128, 16, "e4m3", "bf16", LENS, pool_pages=80)
    case = host_case(w, 91, poison=True)
    out0, lse0, _ = run_hip(to_device(case))
    P = case["kv"].shape[2]
    tok = dict(case)
    tok["k_scale"] = np.ascontiguousarray(np.repeat(case["k_scale"][:, :, None], P, axis=2))
    tok["v_scale"] = np.ascontiguousarray(np.repeat(case["v_scale"][:, :, None], P, axis=2))
    tok["workload"] = custom_workload(len(LENS), 16, 2, 128, 16, "e4m3", "bf16", LENS,
                                      pool_pages=80, kv_scale="token")
    out1, lse1, _ = run_hip(to_device(tok))
    assert torch.allclose(out0, out1, atol=1e-5, rtol=0)
    assert torch.allclose(lse0, lse1, atol=1e-5, rtol=0)


def test_full_size_rowwise_sampled_requests():
    name = "fp8_rowwise_e4m3"
    w = CONFIGS[name]
    seed = list(CONFIGS).index(name) + 1
    _say("full-size", name, "seed", seed)
    dc = device_case(w, seed, "cuda:0", poison=True)
    out, lse, info = run_hip(dc)
    _say("plan", info)
    o = out_to_f64(out)
    assert np.all(np.isfinite(o))
    lens = dc["kv_lens"]
    rows = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5})
    for r in rows:
        sub = sample_request_case(dc, r)
        ref_out, ref_lse = oracle_for(sub)
        _say("  row", r, "len", int(lens[r]))
        compare(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, "e4m3")
    del dc
    torch.cuda.empty_cache()
