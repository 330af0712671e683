"""fp16 KV (with fp16 queries) on the GPU against the oracle: both
contractions on fp16 MFMA, same 2e-3 max-abs tolerance as bf16 KV; fp16
output adds half an ulp of rounding."""
import numpy as np
import pytest
import torch

from gpu_helpers import compare, oracle_for, out_to_f64, run_hip, sample_request_case, to_device
from workloads import CONFIGS, custom_workload, device_case, host_case

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 100, 333, 700, 64, 3]


def _say(*a):
    print("[gpu-f16]", *a, flush=True)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_small_ragged_f16(g, split):
    w = custom_workload(len(LENS), 2 * g, 2, 128, 16, "f16", "f16", LENS,
                        pool_pages=sum(-(-x // 16) for x in LENS) + 7)
    case = host_case(w, 700 + g, poison=True)
    _say("small", g, split)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=64, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(to_device(case), **kw)
    if split == "forced":
        assert info["num_split_requests"] > 0
    compare(out, lse, ref_out, ref_lse, "f16")


@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_f16_page_sizes_and_output(P):
    lens = [1, P, P + 1, 3 * P + 5, 257]
    w = custom_workload(len(lens), 8, 2, 128, P, "f16", "f16", lens,
                        pool_pages=sum(-(-x // P) for x in lens) + 3)
    case = host_case(w, 80 + P, poison=True)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "f16")
        out16, lse16, _ = run_hip(to_device(case), out_dtype="f16", **kw)
        assert out16.dtype == torch.float16
        compare(out16, lse16, ref_out, ref_lse, "f16", out_dtype="f16")


def test_f16_several_new_tokens():
    lens, nq = [40, 333, 17, 100], [30, 7, 4, 16]
    w = custom_workload(4, 16, 4, 128, 16, "f16", "f16", lens, pool_pages=40, qo_lens=nq)
    case = host_case(w, 88, poison=True)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=64, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "f16")


def test_full_size_f16_sampled_requests():
    name = "llama3_8b_f16"
    w = CONFIGS[name]
    seed = list(CONFIGS).index(name) + 1
    _say("full-size", name, "seed", seed)
    dc = device_case(w, seed, "cuda:0", poison=True)
    out, lse, info = run_hip(dc)
    assert np.all(np.isfinite(out_to_f64(out)))
    for r in (0, 21, w.batch - 1):
        sub = sample_request_case(dc, r)
        ref_out, ref_lse = oracle_for(sub)
        compare(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, "f16")
    del dc
    torch.cuda.empty_cache()
