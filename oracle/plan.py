"""The work-partition rule of ``plan()``, stated in plain integer Python.

The pages give the goal, not the rule: FlashDecoding launches blocks over
batch x heads x a split factor along the KV axis ("FlashDecoding + FlashInfer —
the decode-time attention story", §"FlashDecoding — the split-KV trick"), and
FlashInfer balances decode work across CTAs so that the longest sequence does
not stall a batch of mixed short and long sequences (same page, §"What
FlashInfer is", item 3); ``plan()`` does this once per batch shape and ``run()``
reuses it (§"The API you actually use (Python)").

The rule adopted (a reading; the design doc lists it):

1. ``n_r = indptr[r+1] - indptr[r]`` pages and
   ``L_r = (n_r - 1) * P + last_page_len[r]`` tokens per request.
2. With ``S = sum_r n_r``, ``N = max_r n_r``, ``H`` work units per item (one
   per KV head) and ``slots`` workgroups resident on the device at once:

   * a batch of near-equal requests (``8 * N * B <= 9 * S``: the longest is
     within 1/8 of the mean) that already yields at least half the resident
     slots in work units (``2 * B * H >= slots``) is not split: ``C = N``;
     splitting it would add partial states and a merge without evening
     anything out;
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

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import numpy as np


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan(indptr, last_page_len, page_size: int, num_kv_heads: int, slots: int,
         balance: int, min_chunk_pages: int) -> dict:
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
    if slots < 1 or balance < 1 or min_chunk_pages < 1:
        raise ValueError("slots, balance and min_chunk_pages must be positive")

    S = sum(n)
    N = max(n)
    if 8 * N * B <= 9 * S and 2 * B * num_kv_heads >= slots:
        C = N
    else:
        cap = _ceil_div(S * num_kv_heads, slots * balance)
        C = min(N, max(min_chunk_pages, cap))

    G = [_ceil_div(x, C) for x in n]
    merge_indptr = [0]
    for r in range(B):
        merge_indptr.append(merge_indptr[-1] + (G[r] if G[r] > 1 else 0))

    rows = []
    for r in range(B):
        for c in range(G[r]):
            pb = indptr[r] + c * C
            pe = min(pb + C, indptr[r + 1])
            kv_len = (pe - pb) * page_size
            if pe == indptr[r + 1]:
                kv_len -= page_size - last[r]
            slot = merge_indptr[r] + c if G[r] > 1 else -1
            rows.append((r, pb, pe, kv_len, slot, c))
    rows.sort(key=lambda t: (-t[3], t[0], t[5]))
    items = np.array([t[:5] for t in rows], dtype=np.int32).reshape(-1, 5)
    split = np.array([r for r in range(B) if G[r] > 1], dtype=np.int32)
    return {
        "chunk_pages": C,
        "items": items,
        "merge_indptr": np.array(merge_indptr, dtype=np.int32),
        "split_requests": split,
        "num_partials": merge_indptr[-1],
        "kv_lens": np.array([(n[r] - 1) * page_size + last[r] for r in range(B)], dtype=np.int64),
    }
