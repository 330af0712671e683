"""The definition of batched paged-KV decode attention, in float64.

What is computed follows "FlashDecoding + FlashInfer — the decode-time
attention story": one query token per sequence attends over that sequence's
N keys/values (§"FlashDecoding — the split-KV trick", Q of shape (B, H, 1, D));
K/V live in fixed-size pages of shape (num_pages, block_size, num_kv_heads,
head_dim) and a per-request page list with the last page's fill selects them
(§"Paged attention (vLLM)"); query heads share KV heads when num_kv_heads is
smaller than num_qo_heads (§"The API you actually use (Python)").

Readings taken where the pages are silent:

* Request r owns pages ``indices[indptr[r]:indptr[r+1]]`` (n_r >= 1 of them)
  and holds ``L_r = (n_r - 1) * page_size + last_page_len[r]`` tokens; token t
  sits in page ``indices[indptr[r] + t // page_size]`` at slot
  ``t % page_size``.
* Query head h reads KV head ``h // (num_qo_heads // num_kv_heads)``.
* Scores are ``sm_scale * q . k`` with ``sm_scale = 1/sqrt(head_dim)`` unless
  given; no position encoding is applied (the wrapper's
  ``pos_encoding_mode="NONE"``).
* The output is the max-subtracted softmax average of V, and the optional
  log-sum-exp is ``m + ln(d)`` in natural log.
* Several query tokens per request (the "handful with speculative decoding"
  of the page's opening, laid out as the ragged ``qo_indptr`` rows of
  §"Ragged attention — variable-length batching"): the n new tokens of a
  request are its last n KV tokens, in order, and new token i (0-based) sees
  the KV tokens up to and including its own position, i.e. the first
  ``L_r - n + 1 + i`` of them (causal within the new tokens).
* Cascade attention over a shared prefix (the "Cascade Attention" operator
  of "GitHub Spotlight: FlashInfer", §"Core Superpowers: Breaking Down the
  Feature Set", used for shared prompt prefixes in §"Real-World Deployment
  Scenarios", Scenario A): the queries of every request that shares a
  prefix attend to it as one batch, so there the rows are not causal
  (``causal=False``: every row sees all of its request's tokens). The
  cascade's result is plain decode over prefix + suffix, which
  ``merge.merge_normalized`` reaches from the two levels.

The full softmax over each request's gathered tokens is materialised; no
tiling, splitting or reordering is done here (``oracle.merge`` holds the split
form, which tests compare with this one).

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from . import e2m1, int4
from .storage import widen


def request_length(indptr, last_page_len, page_size: int, r: int) -> int:
    n = int(indptr[r + 1]) - int(indptr[r])
    return (n - 1) * page_size + int(last_page_len[r])


def token_locations(indptr, indices, last_page_len, page_size: int, r: int):
    """(page id, slot) of every token of request r, in logical order."""
    L = request_length(indptr, last_page_len, page_size, r)
    t = np.arange(L, dtype=np.int64)
    pages = np.asarray(indices[int(indptr[r]):int(indptr[r + 1])], dtype=np.int64)
    return pages[t // page_size], t % page_size


def gather_request(kv, indptr, indices, last_page_len, r: int, kv_head: int, kv_dtype: str,
                   k_scale=None, v_scale=None):
    """K and V of request r and one KV head as float64 ``[L_r, head_dim]`` each.

    ``kv`` is the combined NHD pool ``[num_pages, 2, page_size, Hkv, D]`` in
    raw storage; index 0 of axis 1 is K, 1 is V. e4m3 scales are
    ``[num_pages, Hkv]`` (one per page and KV head) or ``[num_pages, Hkv,
    page_size]`` (one per token and KV head: the row-wise scaling of
    "FlashInfer vs FlashAttention-3: GPU Kernel Optimization & FP8 Serving
    Latency", §"Production War Story"). e2m1 and int4 rows hold two codes
    per byte (``[..., D/2]``) and their scales are per channel, ``[Hkv, D]``.
    """
    page_size = kv.shape[2]
    page, slot = token_locations(indptr, indices, last_page_len, page_size, r)
    if kv_dtype in ("e2m1", "i4"):
        # packed rows [L, D/2] -> [L, D], times the per-channel scale of the head
        dec = e2m1.decode_packed if kv_dtype == "e2m1" else int4.decode_packed
        ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
        vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)
        K = dec(kv[page, 0, slot, kv_head, :]) * ks[kv_head][None, :]
        V = dec(kv[page, 1, slot, kv_head, :]) * vs[kv_head][None, :]
        return K, V
    K = widen(kv[page, 0, slot, kv_head, :], kv_dtype)
    V = widen(kv[page, 1, slot, kv_head, :], kv_dtype)
    if kv_dtype == "e4m3":
        ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
        vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)
        if ks.ndim == 3:  # one scale per (page, KV head, slot): row-wise
            K = K * ks[page, kv_head, slot][:, None]
            V = V * vs[page, kv_head, slot][:, None]
        else:  # one scale per (page, KV head)
            K = K * ks[page, kv_head][:, None]
            V = V * vs[page, kv_head][:, None]
    return K, V


def attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Softmax attention of one float64 query row over dense float64 K/V."""
    s = sm_scale * (K @ qh)
    m = s.max()
    p = np.exp(s - m)
    d = p.sum()
    return (p @ V) / d, m + math.log(d)


def visible_tokens(L: int, n_new: int, i: int) -> int:
    """KV tokens seen by new token i of a request of L tokens whose last n_new
    tokens are new: all tokens up to and including its own position."""
    return L - n_new + 1 + i


def decode(q, kv, indptr, indices, last_page_len, *, num_kv_heads: int, q_dtype: str,
           kv_dtype: str, sm_scale: Optional[float] = None, k_scale=None, v_scale=None,
           requests: Optional[Iterable[int]] = None, qo_indptr=None, causal: bool = True):
    """Decode attention for every (query token, query head).

    Without ``qo_indptr`` q holds one token per request (``[B, Hq, D]``). With
    it, request r owns q rows ``qo_indptr[r]:qo_indptr[r+1]`` (at least one, at
    most ``L_r``), attended causally as described in the module docstring.
    Returns ``out`` float64 ``[rows, Hq, D]`` and ``lse`` float64 ``[rows, Hq]``.
    With ``requests`` given, only those requests' rows are computed (the rest
    are NaN).
    """
    q64 = widen(q, q_dtype)
    R, Hq, D = q64.shape
    B = len(last_page_len)
    qo = np.arange(B + 1) if qo_indptr is None else np.asarray(qo_indptr, dtype=np.int64)
    if len(qo) != B + 1 or qo[0] != 0 or qo[-1] != R or np.any(np.diff(qo) < 1):
        raise ValueError("qo_indptr must start at 0, give every request a query row and "
                         "end at the number of q rows")
    if Hq % num_kv_heads:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    g = Hq // num_kv_heads
    scale = (1.0 / math.sqrt(D)) if sm_scale is None else float(sm_scale)
    out = np.full((R, Hq, D), np.nan)
    lse = np.full((R, Hq), np.nan)
    for r in (range(B) if requests is None else requests):
        L = request_length(indptr, last_page_len, kv.shape[2], r)
        n_new = int(qo[r + 1] - qo[r])
        if causal and n_new > L:
            raise ValueError("a request has more query tokens than KV tokens")
        for kvh in range(num_kv_heads):
            K, V = gather_request(kv, indptr, indices, last_page_len, r, kvh, kv_dtype,
                                  k_scale, v_scale)
            for i in range(n_new):
                vis = visible_tokens(L, n_new, i) if causal else L
                row = int(qo[r]) + i
                for h in range(kvh * g, (kvh + 1) * g):
                    out[row, h], lse[row, h] = attend(q64[row, h], K[:vis], V[:vis], scale)
    return out, lse


def decode_case(case: dict, requests=None, sm_scale=None):
    """``decode`` on a dict produced by ``workloads.host_case``."""
    w = case["workload"]
    return decode(case["q"], case["kv"], case["indptr"], case["indices"], case["last_page_len"],
                  num_kv_heads=w.num_kv_heads, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                  sm_scale=w.scale() if sm_scale is None else sm_scale,
                  k_scale=case.get("k_scale"), v_scale=case.get("v_scale"), requests=requests,
                  qo_indptr=case.get("qo_indptr"))
