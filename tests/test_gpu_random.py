"""Seeded random configurations against the oracle.

Each case draws a KV format (fp32, bf16, fp16, e4m3 with per-page or per-token
scales, e2m1 or int4), a query/KV head layout (group 1-32, 1-4 KV heads: single heads
and pairs), a page size, ragged lengths (page-aligned and not), one or several
new tokens per request, an automatic or forced split and an output dtype, and
compares the HIP path with the oracle at the format's tolerance.
"""
import numpy as np
import pytest

from gpu_helpers import compare, oracle_for, run_hip, to_device
from workloads import custom_workload, host_case

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw_case(seed: int) -> dict:
    """The configuration of case `seed` (host only; also used by a CPU test)."""
    rng = np.random.default_rng([seed, 20260])
    kv = str(rng.choice(["f32", "bf16", "f16", "e4m3", "e4m3t", "e2m1"]))
    kv_scale = "token" if kv == "e4m3t" else "page"
    kv = "e4m3" if kv == "e4m3t" else kv
    # half of the 4-bit cases are int4 (a stream of its own, so that the other
    # cases' draws do not move)
    if kv == "e2m1" and np.random.default_rng([seed, 4]).random() < 0.5:
        kv = "i4"
    mfma = kv in ("bf16", "f16", "e2m1", "i4") or (kv == "e4m3" and (kv_scale == "token" or rng.random() < 0.7))
    if kv == "f32":
        mfma = False
    d = 128 if (mfma or rng.random() < 0.5) else 64
    if mfma:
        qd = "f16" if kv == "f16" else "bf16"
        g = int(rng.choice([1, 2, 4, 8, 16] + ([32] if kv not in ("e2m1", "i4") else [])))
    else:
        qd = "f32" if kv == "f32" else str(rng.choice(["f32", "bf16"]))
        g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 5))
    P = int(rng.choice([1, 2, 4, 8, 16, 16, 32, 64]))
    B = int(rng.integers(1, 10))
    lens = []
    for _ in range(B):
        if rng.random() < 0.3:
            lens.append(int(P * rng.integers(1, 12)))
        else:
            lens.append(int(rng.integers(1, 600)))
    qo = None
    if mfma and rng.random() < 0.35:
        qo = [int(rng.integers(1, min(L, 20) + 1)) for L in lens]
    split = bool(rng.random() < 0.5)
    out = str(rng.choice(["f32", "bf16", "f16"]))
    return dict(kv=kv, kv_scale=kv_scale, qd=qd, d=d, g=g, hkv=hkv, P=P, lens=lens, qo=qo,
                split=split, out=out)


def build(seed: int):
    c = draw_case(seed)
    pool = sum(-(-L // c["P"]) for L in c["lens"]) + 3
    w = custom_workload(len(c["lens"]), c["g"] * c["hkv"], c["hkv"], c["d"], c["P"], c["kv"],
                        c["qd"], c["lens"], pool_pages=pool, qo_lens=c["qo"],
                        kv_scale=c["kv_scale"])
    return c, w, host_case(w, 4000 + seed, poison=True)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    c, w, case = build(seed)
    print("[gpu-random]", seed, c, flush=True)
    ref_out, ref_lse = oracle_for(case)
    kw = dict(slots=16, balance=1, min_chunk_pages=1) if c["split"] else {}
    out, lse, _ = run_hip(to_device(case), out_dtype=c["out"], **kw)
    compare(out, lse, ref_out, ref_lse, c["kv"], out_dtype=c["out"])


N_LARGE = 12


def draw_large_case(seed: int) -> dict:
    """A batch of 150-1050 short requests on an MFMA form with the device's
    default plan: mostly more work units than resident workgroups, so the
    16-bit and per-page e4m3 forms run persistent launches and the others
    grids of several rounds."""
    rng = np.random.default_rng([seed, 77001])
    kv = str(rng.choice(["bf16", "f16", "e4m3", "e4m3t", "e2m1", "i4"]))
    kv_scale = "token" if kv == "e4m3t" else "page"
    kv = "e4m3" if kv == "e4m3t" else kv
    qd = "f16" if kv == "f16" else "bf16"
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([2, 4, 8]))
    P = int(rng.choice([16, 32]))
    B = int(rng.integers(150, 351)) * (3 if hkv == 2 else 1)  # two heads: one unit per item
    lens = [int(x) for x in rng.integers(1, 300, size=B)]
    qo = None
    if rng.random() < 0.3:
        qo = [int(rng.integers(1, min(L, 4) + 1)) for L in lens]
    return dict(kv=kv, kv_scale=kv_scale, qd=qd, d=128, g=g, hkv=hkv, P=P, lens=lens, qo=qo)


@pytest.mark.parametrize("seed", range(N_LARGE))
def test_random_large_batch(seed):
    c = draw_large_case(seed)
    pool = sum(-(-L // c["P"]) for L in c["lens"]) + 3
    w = custom_workload(len(c["lens"]), c["g"] * c["hkv"], c["hkv"], c["d"], c["P"], c["kv"],
                        c["qd"], c["lens"], pool_pages=pool, qo_lens=c["qo"],
                        kv_scale=c["kv_scale"])
    case = host_case(w, 9000 + seed, poison=True)
    print("[gpu-random-large]", seed, {k: v for k, v in c.items() if k != "lens"},
          "B", len(c["lens"]), flush=True)
    ref_out, ref_lse = oracle_for(case)
    out, lse, info = run_hip(to_device(case))
    print("[gpu-random-large]", seed, "units", info["num_items"] * info["units_per_item"],
          "slots", info["slots"], flush=True)
    compare(out, lse, ref_out, ref_lse, c["kv"])
