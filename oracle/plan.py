"""The work-partition rule of ``plan()``, stated in plain integer Python.

The pages give the goal, not the rule: FlashDecoding launches blocks over
batch x heads x a split factor along the KV axis ("FlashDecoding + FlashInfer —
the decode-time attention story", §"FlashDecoding — the split-KV trick"), and
FlashInfer balances decode work across CTAs so that the longest sequence does
not stall a batch of mixed short and long sequences (same page, §"What
FlashInfer is", item 3); ``plan()`` does this once per batch shape and ``run()``
reuses it (§"The API you actually use (Python)").

The rule adopted (a reading of the pages, not a rule they state):

1. ``n_r = indptr[r+1] - indptr[r]`` pages and
   ``L_r = (n_r - 1) * P + last_page_len[r]`` tokens per request.
2. With ``S = sum_r n_r``, ``N = max_r n_r``, ``H`` work units per item (the
   workgroups one item runs as: one per KV head, or per pair of KV heads),
   ``slots`` workgroups resident on the device at once and ``slots_per_cu``
   of them on one compute unit:

   * a batch of near-equal requests (``8 * N * B <= 9 * S``: the longest is
     within 1/8 of the mean) is cut into ``k`` chunks per request,
     ``C = ceil(N / k)``, where ``k`` in ``[1, max(1, N // C_min)]``
     minimises ``ceil(B * H * k / (CUs * balance)) * (ceil(N / k) + 2 * C_min)``
     (the number of waves of equal work units over the compute units,
     ``CUs = ceil(slots / slots_per_cu)``, times one unit's pages plus
     ``2 * C_min`` pages standing for a workgroup's start and its share of
     the merge), the smallest such ``k`` on ties: equal requests that already
     fill the device stay whole, fewer are cut just enough to fill it;
   * otherwise ``C = min(N, max(C_min, ceil(S * H / (slots * balance))))``:
     no work unit is longer than ``1/balance`` of a slot's fair share of the
     batch, nor shorter than ``C_min`` pages (which bounds the partial-state
     traffic), and nothing is split that fits in one chunk.
3. Request r becomes ``G_r = ceil(n_r / C)`` items; chunk c covers pages
   ``[indptr[r] + c*C, min(indptr[r] + (c+1)*C, indptr[r+1]))``; its token count
   drops ``P - last_page_len[r]`` when it holds the request's last page.
4. ``merge_indptr[r+1] = merge_indptr[r] + (G_r if G_r > 1 else 0)``; item
   (r, c) of a split request writes partial slot ``merge_indptr[r] + c``, an
   unsplit request's single item writes the output directly (slot -1).
5. Items are ordered longest first (descending token count), ties by request
   then chunk index, so the hardware's in-order dispatch starts the long
   work units first and the short ones fill in behind them.

Several new tokens per request (``qo_indptr``, ``q_r`` tokens for request r;
the causal reading is stated in ``oracle.attention``): a work item carries at
most ``queries_per_item`` (``Q``) of a request's new tokens, so request r
counts as ``U_r = ceil(q_r / Q)`` units of ``n_r`` pages each. Steps 2-5 run
over units instead of requests (``B`` = number of units, ``S`` = sum of their
pages; with one token per request nothing changes), every chunk of a request
is repeated for each of its query blocks (block b holds tokens
``[b*Q, min((b+1)*Q, q_r))``), and partial states are kept per query token:
``merge_indptr[r+1] = merge_indptr[r] + (G_r * q_r if G_r > 1 else 0)``, item
(r, c, b) writes rows ``merge_indptr[r] + c*q_r + b*Q + i`` for its block's
token i. Each item also records its first q row ``qo_indptr[r] + b*Q``, its
token count, and how many of its KV tokens the block's first token sees,
``min(kv_len, L_r - q_r + 1 + b*Q - c*C*P)`` (token i of the block sees
``min(kv_len, that + i)``; a value <= 0 means it sees none). Ties in step 5
go by request, chunk, then query block. With ``causal=False`` (the shared
prefix of cascade attention) every row sees the whole item (``visible =
kv_len``) and a request may have more query rows than KV tokens.

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import numpy as np


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


ITEM_COLUMNS = ("request", "page_begin", "page_end", "kv_len", "partial_slot", "q_row",
                "q_len", "visible")


def plan(indptr, last_page_len, page_size: int, num_kv_heads: int, slots: int,
         balance: int, min_chunk_pages: int, qo_indptr=None, queries_per_item: int = 1,
         causal: bool = True, slots_per_cu: int = 1) -> dict:
    indptr = [int(x) for x in indptr]
    last = [int(x) for x in last_page_len]
    B = len(last)
    if B < 1:
        raise ValueError("the batch needs at least one request")
    if len(indptr) != B + 1 or indptr[0] != 0:
        raise ValueError("indptr must have batch+1 entries starting at 0")
    n = [indptr[r + 1] - indptr[r] for r in range(B)]
    if any(x < 1 for x in n):
        raise ValueError("every request needs at least one page")
    if any(not (1 <= lp <= page_size) for lp in last):
        raise ValueError("last_page_len must lie in [1, page_size]")
    if slots < 1 or balance < 1 or min_chunk_pages < 1 or queries_per_item < 1:
        raise ValueError("slots, balance, min_chunk_pages and queries_per_item must be positive")
    L = [(n[r] - 1) * page_size + last[r] for r in range(B)]
    qo = list(range(B + 1)) if qo_indptr is None else [int(x) for x in qo_indptr]
    if len(qo) != B + 1 or qo[0] != 0:
        raise ValueError("qo_indptr must have batch+1 entries starting at 0")
    nq = [qo[r + 1] - qo[r] for r in range(B)]
    if any(nq[r] < 1 or (causal and nq[r] > L[r]) for r in range(B)):
        raise ValueError("every request needs at least 1 (causal: at most L_r) query tokens")
    Q = queries_per_item
    U = [_ceil_div(x, Q) for x in nq]  # query blocks (units) per request

    units = sum(U)
    S = sum(n[r] * U[r] for r in range(B))
    N = max(n)
    if 8 * N * units <= 9 * S:
        best_k, best_cost = 1, None
        for k in range(1, max(1, N // min_chunk_pages) + 1):
            waves = _ceil_div(units * num_kv_heads * k,
                              _ceil_div(slots, max(1, slots_per_cu)) * balance)
            cost = waves * (_ceil_div(N, k) + 2 * min_chunk_pages)
            if best_cost is None or cost < best_cost:
                best_k, best_cost = k, cost
        C = _ceil_div(N, best_k)
    else:
        cap = _ceil_div(S * num_kv_heads, slots * balance)
        C = min(N, max(min_chunk_pages, cap))

    G = [_ceil_div(x, C) for x in n]
    merge_indptr = [0]
    for r in range(B):
        merge_indptr.append(merge_indptr[-1] + (G[r] * nq[r] if G[r] > 1 else 0))

    rows = []
    for r in range(B):
        for c in range(G[r]):
            pb = indptr[r] + c * C
            pe = min(pb + C, indptr[r + 1])
            kv_len = (pe - pb) * page_size
            if pe == indptr[r + 1]:
                kv_len -= page_size - last[r]
            for b in range(U[r]):
                q_len = min(Q, nq[r] - b * Q)
                visible = min(kv_len, L[r] - nq[r] + 1 + b * Q - c * C * page_size)
                if not causal:
                    visible = kv_len
                slot = merge_indptr[r] + c * nq[r] + b * Q if G[r] > 1 else -1
                rows.append((r, pb, pe, kv_len, slot, qo[r] + b * Q, q_len, visible, c, b))
    rows.sort(key=lambda t: (-t[3], t[0], t[8], t[9]))
    items = np.array([t[:8] for t in rows], dtype=np.int32).reshape(-1, len(ITEM_COLUMNS))
    split = np.array([r for r in range(B) if G[r] > 1], dtype=np.int32)
    return {
        "chunk_pages": C,
        "items": items,
        "merge_indptr": np.array(merge_indptr, dtype=np.int32),
        "split_requests": split,
        "num_partials": merge_indptr[-1],
        "kv_lens": np.array(L, dtype=np.int64),
    }
