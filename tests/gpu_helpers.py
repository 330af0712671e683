"""Shared helpers for the GPU parity tests: move seeded host cases to the
device, run the HIP path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_decode_plan_amd as pk
from oracle import attention

# e2m1 and int4 are compared against the same dequantised values with the
# arithmetic of the bf16 path (exact widening, fp32 accumulation), so they keep
# 2e-3.
TOL = {"f32": 2e-3, "bf16": 2e-3, "f16": 2e-3, "e4m3": 3e-2, "e2m1": 2e-3, "i4": 2e-3}
DEV = "cuda:0"


def to_device(case: dict, device=DEV) -> dict:
    w = case["workload"]
    if w.q_dtype == "bf16":
        q = torch.from_numpy(case["q"].view(np.int16)).view(torch.bfloat16)
    else:
        q = torch.from_numpy(case["q"])
    kv = case["kv"]
    if w.kv_dtype == "bf16":
        kvt = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16)
    else:
        kvt = torch.from_numpy(np.ascontiguousarray(kv))
    d = {
        "q": q.to(device).contiguous(),
        "kv": kvt.to(device).contiguous(),
        "indptr": case["indptr"],
        "indices": torch.from_numpy(case["indices"]).to(device),
        "last_page_len": case["last_page_len"],
        "k_scale": None,
        "v_scale": None,
        "workload": w,
        "qo_indptr": case.get("qo_indptr"),
    }
    if w.kv_dtype in ("e4m3", "e2m1", "i4"):
        d["k_scale"] = torch.from_numpy(case["k_scale"]).to(device).contiguous()
        d["v_scale"] = torch.from_numpy(case["v_scale"]).to(device).contiguous()
    return d


_WS = {}


def workspace(nbytes=pk.DEFAULT_WORKSPACE_BYTES, device=DEV):
    key = (device, nbytes)
    if key not in _WS:
        _WS[key] = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return _WS[key]


def run_hip(dcase: dict, out_dtype="f32", slots=0, balance=0, min_chunk_pages=0, lse=True,
            ws_bytes=pk.DEFAULT_WORKSPACE_BYTES, kv=None, indices=None):
    w = dcase["workload"]
    wrapper = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(ws_bytes), "NHD")
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    wrapper.plan(dcase["indptr"], dcase["indices"] if indices is None else indices,
                 dcase["last_page_len"], w.num_qo_heads, w.num_kv_heads, w.head_dim,
                 w.page_size, q_data_type=dcase["q"].dtype,
                 kv_data_type=(w.kv_dtype if w.kv_dtype in ("e4m3", "e2m1", "i4")
                               else dcase["kv"].dtype),
                 out_data_type=odt, sm_scale=w.scale(), slots=slots, balance=balance,
                 min_chunk_pages=min_chunk_pages, qo_indptr=dcase.get("qo_indptr"),
                 kv_scale=w.kv_scale)
    out, l = wrapper.run(dcase["q"], dcase["kv"] if kv is None else kv, return_lse=lse,
                         k_scale=dcase["k_scale"], v_scale=dcase["v_scale"])
    torch.cuda.synchronize()
    info = wrapper.plan_info
    wrapper.close()
    return out, l, info


def out_to_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def compare(out, lse, ref_out, ref_lse, kv_dtype, out_dtype="f32", rows=None):
    """Max-abs error check at the tolerance for the KV dtype (bf16 output adds
    its own rounding, half an ulp of the reference)."""
    o = out_to_f64(out)
    if rows is not None:
        o = o[rows]
        ref_out = ref_out[rows]
    assert np.all(np.isfinite(o)), "non-finite output"
    tol = TOL[kv_dtype]
    err = np.abs(o - ref_out)
    bound = tol + (np.abs(ref_out) * {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}.get(out_dtype, 0.0))
    worst = float(err.max())
    assert np.all(err <= bound), f"max-abs error {worst:.3e} above tolerance {tol}"
    if lse is not None:
        lv = lse.cpu().numpy().astype(np.float64)
        rl = ref_lse
        if rows is not None:
            lv, rl = lv[rows], rl[rows]
        lerr = float(np.abs(lv - rl).max())
        assert lerr <= tol, f"lse error {lerr:.3e}"
    return worst


def oracle_for(case: dict, requests=None):
    return attention.decode_case(case, requests=requests)


def sample_request_case(dcase: dict, r: int) -> dict:
    """Host copy of one request's pages from a device case, renumbered, for the oracle."""
    w = dcase["workload"]
    indptr, last = dcase["indptr"], dcase["last_page_len"]
    idx = dcase["indices"]
    if isinstance(idx, torch.Tensor):
        idx = idx.cpu().numpy()
    pages = torch.as_tensor(np.asarray(idx[int(indptr[r]):int(indptr[r + 1])], dtype=np.int64),
                            device=dcase["kv"].device)
    kv = dcase["kv"].index_select(0, pages)
    if w.kv_dtype == "bf16":
        kvh = kv.view(torch.int16).cpu().numpy().view(np.uint16)
    elif w.kv_dtype in ("f32", "f16"):
        kvh = kv.cpu().numpy()
    else:
        kvh = kv.cpu().numpy().view(np.uint8)
    qo = dcase.get("qo_indptr")
    q0, q1 = (r, r + 1) if qo is None else (int(qo[r]), int(qo[r + 1]))
    q = dcase["q"][q0:q1]
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16) if w.q_dtype == "bf16" else q.cpu().numpy()
    n = len(pages)
    sub = {
        "q": qh, "kv": kvh,
        "indptr": np.array([0, n], np.int32),
        "indices": np.arange(n, dtype=np.int32),
        "last_page_len": np.array([last[r]], np.int32),
        "num_pages": n,
        "workload": w,
        "k_scale": None, "v_scale": None,
        "qo_indptr": None if qo is None else np.array([0, q1 - q0], np.int32),
    }
    if w.kv_dtype == "e4m3":
        sub["k_scale"] = dcase["k_scale"].index_select(0, pages).cpu().numpy()
        sub["v_scale"] = dcase["v_scale"].index_select(0, pages).cpu().numpy()
    elif w.kv_dtype in ("e2m1", "i4"):  # per channel: not tied to pages
        sub["k_scale"] = dcase["k_scale"].cpu().numpy()
        sub["v_scale"] = dcase["v_scale"].cpu().numpy()
    return sub
