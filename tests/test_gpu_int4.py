"""int4 KV (two's complement) with per-channel scales on the GPU against the oracle.

K and V are packed signed 4-bit codes (two per byte) with one fp32 scale per
(KV head, channel) each; the oracle decodes the codes by their definition and
multiplies by the scales in float64. The kernel widens (code + 8) * 2^-9 to
bf16 exactly, removes the offset from the scores and the output, and
accumulates in fp32, so the bf16 tolerance (2e-3 max-abs) applies.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import compare, oracle_for, out_to_f64, run_hip, sample_request_case, to_device
from oracle import int4
from workloads import CONFIGS, custom_workload, device_case, host_case

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 100, 333, 700, 64, 3]


def _say(*a):
    print("[gpu-int4]", *a, flush=True)


def _pool(lens, P, extra):
    return sum(-(-x // P) for x in lens) + extra


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("split", ["auto", "forced"])
def test_small_ragged_int4(g, split):
    w = custom_workload(len(LENS), 2 * g, 2, 128, 16, "i4", "bf16", LENS,
                        pool_pages=_pool(LENS, 16, 7))
    case = host_case(w, 1700 + g, poison=True)
    _say("small", g, split)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=64, balance=1, min_chunk_pages=1) if split == "forced" else {}
    out, lse, info = run_hip(to_device(case), **kw)
    if split == "forced":
        assert info["num_split_requests"] > 0
    compare(out, lse, ref_out, ref_lse, "i4")


HEADS_PER_WG = {1: 1, 2: 2, 3: 1, 4: 2, 8: 2}


@pytest.mark.parametrize("hkv", sorted(HEADS_PER_WG))
def test_int4_kv_head_counts(hkv):
    """One KV head or a pair of KV heads per workgroup, against the oracle."""
    w = custom_workload(len(LENS), 4 * hkv, hkv, 128, 16, "i4", "bf16", LENS,
                        pool_pages=_pool(LENS, 16, 5))
    case = host_case(w, 1900 + hkv, poison=True)
    _say("kv heads", hkv)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=64, balance=1, min_chunk_pages=1)):
        out, lse, info = run_hip(to_device(case), **kw)
        assert info["units_per_item"] == hkv // HEADS_PER_WG[hkv]
        compare(out, lse, ref_out, ref_lse, "i4")


@pytest.mark.parametrize("P", [1, 2, 4, 8, 16, 32, 64])
def test_int4_page_sizes(P):
    lens = [1, P, P + 1, 3 * P + 5, 257]
    w = custom_workload(len(lens), 8, 2, 128, P, "i4", "bf16", lens,
                        pool_pages=_pool(lens, P, 3))
    case = host_case(w, 180 + P, poison=True)
    _say("pages", P)
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=8, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "i4")


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_int4_16bit_outputs(out_dtype):
    w = custom_workload(len(LENS), 8, 2, 128, 16, "i4", "bf16", LENS,
                        pool_pages=_pool(LENS, 16, 2))
    case = host_case(w, 193, poison=True)
    ref_out, ref_lse = oracle_for(case)
    out, lse, _ = run_hip(to_device(case), out_dtype=out_dtype)
    compare(out, lse, ref_out, ref_lse, "i4", out_dtype=out_dtype)


def test_int4_with_several_new_tokens():
    lens, nq = [40, 333, 17, 100], [30, 7, 4, 16]
    w = custom_workload(4, 16, 4, 128, 16, "i4", "bf16", lens, pool_pages=40, qo_lens=nq)
    case = host_case(w, 179, poison=True)
    _say("several new tokens")
    ref_out, ref_lse = oracle_for(case)
    for kw in ({}, dict(slots=64, balance=1, min_chunk_pages=1)):
        out, lse, _ = run_hip(to_device(case), **kw)
        compare(out, lse, ref_out, ref_lse, "i4")


@pytest.mark.parametrize("fill", [0x88, 0x77, 0x08, 0x80])
def test_int4_extreme_codes(fill):
    """Every V code at an end of the range (-8 or 7, or alternating) and K
    codes random: the offset the kernel adds to the codes must cancel
    exactly; with all V codes equal the output is that code times the
    channel scale."""
    lens = [5, 300, 64]
    w = custom_workload(3, 8, 2, 128, 16, "i4", "bf16", lens, pool_pages=_pool(lens, 16, 1))
    case = host_case(w, 211, poison=False)
    case["kv"] = case["kv"].copy()
    case["kv"][:, 1] = fill
    _say("extreme V codes", hex(fill))
    ref_out, ref_lse = oracle_for(case)
    out, lse, _ = run_hip(to_device(case))
    compare(out, lse, ref_out, ref_lse, "i4")
    if fill in (0x88, 0x77):
        code = int4.value(fill & 0xF)
        vs = case["v_scale"].astype(np.float64)  # [Hkv, D]
        want = np.repeat(code * vs, 4, axis=0)[None]  # q head h reads KV head h // 4
        assert np.allclose(out_to_f64(out), want, atol=2e-3 * max(1.0, np.abs(want).max()), rtol=0)


def test_int4_unit_scales_match_bf16_kv_of_the_decoded_values():
    """With every channel scale 1 the int4 path computes what the bf16 path
    computes on a bf16 pool holding the decoded codes (exact in bf16); the two
    differ only in rounding order and the offset's cancellation."""
    wi = custom_workload(len(LENS), 16, 2, 128, 16, "i4", "bf16", LENS, pool_pages=80)
    case = host_case(wi, 195, poison=False)
    case["k_scale"] = np.ones_like(case["k_scale"])
    case["v_scale"] = np.ones_like(case["v_scale"])
    outi, lsei, _ = run_hip(to_device(case))
    vals = int4.decode_packed(case["kv"]).astype(np.float32)  # exact in bf16 too
    bf = dict(case)
    bf["workload"] = custom_workload(len(LENS), 16, 2, 128, 16, "bf16", "bf16", LENS,
                                     pool_pages=80)
    bf["kv"] = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bf["k_scale"] = bf["v_scale"] = None
    out16, lse16, _ = run_hip(to_device(bf))
    assert torch.allclose(outi, out16, atol=2e-4, rtol=0)
    assert torch.allclose(lsei, lse16, atol=2e-4, rtol=0)


def test_full_size_int4_sampled_requests():
    name = "int4_kv"
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
        compare(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, "i4")
    del dc
    torch.cuda.empty_cache()
