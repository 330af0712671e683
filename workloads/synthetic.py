"""Seeded synthetic decode workloads: page tables, paged KV pools and queries.

Storage conventions (shared by every consumer, so each side decodes the raw
bytes itself):

* ``kv`` is the combined NHD page pool ``[num_pages, 2, page_size,
  num_kv_heads, head_dim]``; index 0 of the second axis holds K, index 1 holds V.
* ``"f32"`` storage is ``float32``, ``"f16"`` storage ``float16``; ``"bf16"`` storage is the raw 16-bit
  pattern as ``uint16``; ``"e4m3"`` storage is the raw OCP E4M3FN byte as
  ``uint8`` with fp32 scales ``k_scale``/``v_scale`` of shape
  ``[num_pages, num_kv_heads]`` (one per page and KV head) or, for a
  workload with ``kv_scale="token"``, ``[num_pages, num_kv_heads,
  page_size]`` (one per token and KV head; a head's scales of a page are
  contiguous). ``"e2m1"`` storage is packed FP4 E2M1 codes as ``uint8``
  ``[num_pages, 2, page_size, num_kv_heads, head_dim / 2]`` (element 2i in the
  low nibble of byte i) with fp32 per-channel scales ``k_scale``/``v_scale``
  of shape ``[num_kv_heads, head_dim]``; ``"i4"`` storage is the same with
  two's-complement int4 codes (-8 .. 7) in the nibbles.
* ``q`` is ``[rows, num_qo_heads, head_dim]`` in ``"f32"`` or ``"bf16"``
  storage: one row per request, or, for a workload with several new tokens
  per request, the ragged rows ``qo_indptr[r]:qo_indptr[r+1]`` of request r
  (``qo_indptr`` int32 ``[batch+1]``; ``None`` for one token per request).
* The page table is ``indptr`` (int32 ``[batch+1]``), ``indices`` (int32 page
  ids) and ``last_page_len`` (int32 ``[batch]``), as in the paged-KV wrapper
  of "FlashDecoding + FlashInfer — the decode-time attention story", §"The API
  you actually use (Python)" and §"Paged attention (vLLM)".

Slots that no request reads (the tail of each last page, and pool pages that
no request references) can be poisoned with NaN (0x7F for e4m3) so that a
kernel reading past a request's end cannot go unnoticed.

The module draws random numbers and converts them to storage formats; it does
no attention arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

KV_DTYPES = ("f32", "bf16", "f16", "e4m3", "e2m1", "i4")
Q_DTYPES = ("f32", "bf16", "f16")
E4M3_MAX = 448.0
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BYTE = 0x7F
E2M1_POISON_BYTE = 0x77  # E2M1 has no NaN: both codes +6, the largest value
I4_POISON_BYTE = 0x77  # int4 has no NaN: both codes +7, the largest value
I4_STEPS_PER_SIGMA = 7.0 / 3.0  # int4 codes: 3 standard deviations of a channel map to 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic decode batch.

    ``context`` is one of ``("fixed", L)``, ``("loguniform", lo, hi)``,
    ``("uniform", lo, hi)`` (inclusive) or ``("list", (L0, L1, ...))``.
    ``pool_pages`` is the size of the page pool; ``None`` means exactly the
    pages the batch uses. Page ids are a random permutation of the pool.
    ``queries`` is ``None`` (one query token per request) or a spec of the
    same kinds as ``context`` for the number of new tokens per request,
    clipped to ``[1, L_r]``.
    ``shared_prefix`` is ``None`` or ``(groups, prefix_tokens)``: the requests
    fall into ``groups`` contiguous, near-equal groups, each sharing one prefix
    of ``prefix_tokens`` tokens (whole pages) ahead of its requests' own
    ``context`` tokens.
    """

    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str
    q_dtype: str
    context: tuple
    pool_pages: Optional[int] = None
    sm_scale: Optional[float] = None
    queries: Optional[tuple] = None
    shared_prefix: Optional[tuple] = None
    kv_scale: str = "page"  # e4m3 scale granularity: "page" (page, head) or "token"

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    # Single sequence: 32 used pages scattered in a 64-page pool, fp32.
    "single_seq_fp32": Workload(
        "single_seq_fp32", 1, 4, 4, 64, 16, "f32", "f32", ("fixed", 512), pool_pages=64),
    # Llama-3-8B-shaped decode: GQA 4, every context 2048, bf16.
    "llama3_8b_bf16": Workload(
        "llama3_8b_bf16", 64, 32, 8, 128, 16, "bf16", "bf16", ("fixed", 2048)),
    # Heterogeneous ragged batch, contexts log-uniform in [256, 65536].
    "ragged_loguniform_bf16": Workload(
        "ragged_loguniform_bf16", 256, 32, 8, 128, 16, "bf16", "bf16",
        ("loguniform", 256, 65536)),
    # Long context, small batch, GQA 8, 64-token pages.
    "long_ctx_gqa8_bf16": Workload(
        "long_ctx_gqa8_bf16", 2, 64, 8, 128, 64, "bf16", "bf16", ("fixed", 131072)),
    # fp8 (E4M3) KV with one fp32 scale per (page, KV head); q bf16.
    "fp8_kv_e4m3": Workload(
        "fp8_kv_e4m3", 128, 32, 8, 128, 16, "e4m3", "bf16", ("uniform", 1024, 32768)),
    # Speculative-style multi-token decode: the Llama-3-8B-shaped batch with 4
    # new tokens per request (16 query rows per KV head).
    "spec4_llama3_8b_bf16": Workload(
        "spec4_llama3_8b_bf16", 64, 32, 8, 128, 16, "bf16", "bf16", ("fixed", 2048),
        queries=("fixed", 4)),
    # fp8 KV with row-wise scales: one fp32 scale per (token, KV head).
    "fp8_rowwise_e4m3": Workload(
        "fp8_rowwise_e4m3", 128, 32, 8, 128, 16, "e4m3", "bf16", ("uniform", 1024, 32768),
        kv_scale="token"),
    # The Llama-3-8B-shaped batch in fp16 (q, KV and output).
    "llama3_8b_f16": Workload(
        "llama3_8b_f16", 64, 32, 8, 128, 16, "f16", "f16", ("fixed", 2048)),
    # FP4 (E2M1) KV with per-channel fp32 scales, the fp8 workload's shape.
    "fp4_kv_e2m1": Workload(
        "fp4_kv_e2m1", 128, 32, 8, 128, 16, "e2m1", "bf16", ("uniform", 1024, 32768)),
    # int4 KV (two's complement) with per-channel fp32 scales, the same shape.
    "int4_kv": Workload(
        "int4_kv", 128, 32, 8, 128, 16, "i4", "bf16", ("uniform", 1024, 32768)),
    # Cascade: 64 requests share one 8192-token prefix (a long system prompt or
    # document) and each has 512 tokens of its own.
    "cascade_prefix8k_bf16": Workload(
        "cascade_prefix8k_bf16", 64, 32, 8, 128, 16, "bf16", "bf16", ("fixed", 512),
        shared_prefix=(1, 8192)),
}
CONFIG_ORDER = list(CONFIGS)


def custom_workload(batch, num_qo_heads, num_kv_heads, head_dim, page_size, kv_dtype,
                    q_dtype, lens: Sequence[int], pool_pages=None, sm_scale=None,
                    name="custom", qo_lens: Optional[Sequence[int]] = None,
                    kv_scale: str = "page") -> Workload:
    queries = None if qo_lens is None else ("list", tuple(int(x) for x in qo_lens))
    return Workload(name, batch, num_qo_heads, num_kv_heads, head_dim, page_size, kv_dtype,
                    q_dtype, ("list", tuple(int(x) for x in lens)), pool_pages, sm_scale,
                    queries, kv_scale=kv_scale)


def _draw_lengths(spec: tuple, batch: int, rng: np.random.Generator) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        return np.full(batch, int(spec[1]), dtype=np.int64)
    if kind == "loguniform":
        lo, hi = spec[1], spec[2]
        x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch)))
        return np.clip(x, lo, hi).astype(np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=batch, endpoint=True).astype(np.int64)
    if kind == "list":
        lens = np.asarray(spec[1], dtype=np.int64)
        assert lens.shape == (batch,)
        return lens
    raise ValueError(f"unknown length kind {kind!r}")


def _context_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    return _draw_lengths(w.context, w.batch, rng)


def query_rows(table: dict) -> int:
    """Number of q rows of a page table (one per request unless ``qo_indptr``)."""
    qo = table.get("qo_indptr")
    return len(table["last_page_len"]) if qo is None else int(qo[-1])


def _shared_prefix_table(w: Workload, seed: int) -> dict:
    """Page tables of a shared-prefix workload: the full per-request lists
    (prefix pages, then the request's own), the prefix level (one request per
    group) and the suffix level (each request's own pages)."""
    rng = np.random.default_rng(seed)
    lens = _context_lengths(w, rng)
    if np.any(lens < 1):
        raise ValueError("every request needs at least one token of its own")
    groups, prefix_tokens = w.shared_prefix
    P = w.page_size
    if prefix_tokens % P or prefix_tokens < P or not 1 <= groups <= w.batch:
        raise ValueError("the shared prefix must be whole pages and groups in [1, batch]")
    npre = prefix_tokens // P
    n = (lens + P - 1) // P
    last = (((lens - 1) % P) + 1).astype(np.int32)
    used = groups * npre + int(n.sum())
    pool = max(int(w.pool_pages or used), used)
    perm = rng.permutation(pool)[:used].astype(np.int32)
    prefixes = [perm[g * npre:(g + 1) * npre] for g in range(groups)]
    at = groups * npre
    own = []
    for r in range(w.batch):
        own.append(perm[at:at + int(n[r])])
        at += int(n[r])
    bounds = np.linspace(0, w.batch, groups + 1).round().astype(np.int32)
    owner = np.searchsorted(bounds, np.arange(w.batch), side="right") - 1

    def table(lists, last_page_len):
        cnt = np.array([len(x) for x in lists], dtype=np.int64)
        indptr = np.zeros(len(lists) + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(cnt)
        return {"indptr": indptr, "indices": np.concatenate(lists).astype(np.int32),
                "last_page_len": np.asarray(last_page_len, dtype=np.int32)}

    full = table([np.concatenate([prefixes[owner[r]], own[r]]) for r in range(w.batch)], last)
    full.update({"kv_lens": (lens + prefix_tokens).astype(np.int64), "num_pages": pool,
                 "qo_indptr": None,
                 "shared": table(prefixes, np.full(groups, P)),
                 "unique": table(own, last),
                 "group_qo_indptr": bounds.astype(np.int32)})
    return full


def page_table(w: Workload, seed: int) -> dict:
    """Draw context lengths and a shuffled page table for ``w``."""
    if w.shared_prefix is not None:
        return _shared_prefix_table(w, seed)
    rng = np.random.default_rng(seed)
    lens = _context_lengths(w, rng)
    if np.any(lens < 1):
        raise ValueError("every request needs at least one token")
    P = w.page_size
    n = (lens + P - 1) // P
    last = ((lens - 1) % P) + 1
    used = int(n.sum())
    pool = max(int(w.pool_pages or used), used)
    indices = rng.permutation(pool)[:used].astype(np.int32)
    indptr = np.zeros(w.batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(n)
    qo_indptr = None
    if w.queries is not None:
        nq = np.clip(_draw_lengths(w.queries, w.batch, np.random.default_rng([seed, 2])), 1, lens)
        qo_indptr = np.zeros(w.batch + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(nq)
    return {
        "indptr": indptr,
        "indices": indices,
        "last_page_len": last.astype(np.int32),
        "kv_lens": lens.astype(np.int64),
        "num_pages": pool,
        "qo_indptr": qo_indptr,
    }


def explicit_table(page_lists: Sequence[Sequence[int]], last_page_len: Sequence[int],
                   page_size: int, num_pages: int) -> dict:
    """A page table written out by hand (ids may repeat across requests)."""
    n = np.array([len(p) for p in page_lists], dtype=np.int64)
    indptr = np.zeros(len(page_lists) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(n)
    indices = np.concatenate([np.asarray(p, dtype=np.int32) for p in page_lists])
    last = np.asarray(last_page_len, dtype=np.int32)
    lens = (n - 1) * page_size + last
    return {"indptr": indptr, "indices": indices, "last_page_len": last,
            "kv_lens": lens.astype(np.int64), "num_pages": int(num_pages), "qo_indptr": None}


def read_mask(table: dict, page_size: int) -> np.ndarray:
    """Boolean ``[num_pages, page_size]``: True where some request reads the slot."""
    mask = np.zeros((table["num_pages"], page_size), dtype=bool)
    indptr, indices, last = table["indptr"], table["indices"], table["last_page_len"]
    for r in range(len(last)):
        pages = indices[indptr[r]:indptr[r + 1]]
        if len(pages) == 0:
            continue
        mask[pages[:-1], :] = True
        mask[pages[-1], : int(last[r])] = True
    return mask


# ---------------------------------------------------------------- host (numpy)

def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.clip(x, -E4M3_MAX, E4M3_MAX), dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _quantize_pool_e4m3(pool32: np.ndarray, per_token: bool = False):
    """Per (page, K/V, KV head) block — or per (page, K/V, token, KV head) row —
    scale = amax / 448, bytes = RNE(x / scale)."""
    if per_token:
        amax = np.abs(pool32).max(axis=4)  # [pages, 2, P, Hkv]
        scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
        y = pool32 / scale[..., None]
        st = np.ascontiguousarray(scale.transpose(0, 1, 3, 2))  # [pages, 2, Hkv, P]
        return _to_e4m3_bytes(y), st[:, 0].copy(), st[:, 1].copy()
    amax = np.abs(pool32).max(axis=(2, 4))  # [pages, 2, Hkv]
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    y = pool32 / scale[:, :, None, :, None]
    return _to_e4m3_bytes(y), scale[:, 0, :].copy(), scale[:, 1, :].copy()


# FP4 E2M1 codes by round-to-nearest-even onto the grid 0, 0.5, 1, 1.5, 2, 3,
# 4, 6 with saturation: the magnitude code is the number of rounding
# boundaries passed; at a boundary the even code (mantissa bit 0) wins, so
# boundaries below an odd code are exclusive and those below an even code
# inclusive.
E2M1_BOUNDS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False),
               (3.5, True), (5.0, False))


def _e2m1_codes(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    idx = np.zeros(y.shape, np.uint8)
    for b, inclusive in E2M1_BOUNDS:
        idx += (a >= b) if inclusive else (a > b)
    return idx | (np.signbit(y).astype(np.uint8) << 3)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _channel_magnitudes(draw, shape):
    """Per-(K/V, KV head, channel) magnitudes m = exp(0.5 z): values are m * z'
    for standard normal z', stored as 4-bit codes of m z' / s: E2M1 with scale
    s = m / 2 (codes saturate at 3 standard deviations of their channel), int4
    with s = 3 m / 7 (7 at 3 standard deviations, round half to even, clipped
    to -8 .. 7)."""
    return np.exp(0.5 * draw(shape))


def host_case(w: Workload, seed: int, poison: bool = True, table: Optional[dict] = None) -> dict:
    """Small-case inputs as numpy storage arrays (see module docstring)."""
    if table is None:
        table = page_table(w, seed)
    rng = np.random.default_rng([seed, 1])
    P, Hkv, D = w.page_size, w.num_kv_heads, w.head_dim
    q32 = rng.standard_normal((query_rows(table), w.num_qo_heads, D), dtype=np.float32)
    pool32 = rng.standard_normal((table["num_pages"], 2, P, Hkv, D), dtype=np.float32)
    k_scale = v_scale = None
    if w.kv_dtype == "f32":
        kv = pool32
    elif w.kv_dtype == "f16":
        kv = pool32.astype(np.float16)
    elif w.kv_dtype == "bf16":
        kv = _to_bf16_bits(pool32)
    elif w.kv_dtype == "e4m3":
        kv, k_scale, v_scale = _quantize_pool_e4m3(pool32, w.kv_scale == "token")
    elif w.kv_dtype == "e2m1":
        m = _channel_magnitudes(lambda sh: rng.standard_normal(sh), (2, Hkv, D))
        scale = (m / 2).astype(np.float32)
        kv = _pack_nibbles(_e2m1_codes(2 * pool32))
        k_scale, v_scale = scale[0].copy(), scale[1].copy()
    elif w.kv_dtype == "i4":
        m = _channel_magnitudes(lambda sh: rng.standard_normal(sh), (2, Hkv, D))
        scale = (m / I4_STEPS_PER_SIGMA).astype(np.float32)
        codes = np.clip(np.rint(pool32 * np.float32(I4_STEPS_PER_SIGMA)), -8, 7).astype(np.int8)
        kv = _pack_nibbles(codes.view(np.uint8) & np.uint8(0xF))
        k_scale, v_scale = scale[0].copy(), scale[1].copy()
    else:
        raise ValueError(w.kv_dtype)
    q = {"f32": q32, "f16": None, "bf16": None}[w.q_dtype]
    if w.q_dtype == "f16":
        q = q32.astype(np.float16)
    elif w.q_dtype == "bf16":
        q = _to_bf16_bits(q32)
    if poison:
        unread = ~read_mask(table, P)
        nan = {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
               "bf16": np.uint16(BF16_NAN_BITS), "e4m3": np.uint8(E4M3_NAN_BYTE),
               "e2m1": np.uint8(E2M1_POISON_BYTE), "i4": np.uint8(I4_POISON_BYTE)}[w.kv_dtype]
        kv = kv.copy()
        kv[:, 0][unread] = nan
        kv[:, 1][unread] = nan
    out = dict(table)
    out.update({"q": q, "kv": kv, "k_scale": k_scale, "v_scale": v_scale, "workload": w})
    return out


# ---------------------------------------------------------------- device (torch)

def device_case(w: Workload, seed: int, device, poison: bool = False,
                table: Optional[dict] = None, chunk_pages: int = 8192) -> dict:
    """Full-size inputs drawn directly in device memory with a seeded torch generator.

    Returns torch tensors: ``q`` (float32 or bfloat16), ``kv`` (float32,
    bfloat16, or uint8 bytes for e4m3 and packed e2m1 / int4),
    ``k_scale``/``v_scale`` (float32, e4m3, e2m1 and int4 only), and the numpy
    page table.
    """
    import torch

    if table is None:
        table = page_table(w, seed)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 7919 + 17)
    P, Hkv, D = w.page_size, w.num_kv_heads, w.head_dim
    npg = table["num_pages"]
    qdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.q_dtype]
    q = torch.randn((query_rows(table), w.num_qo_heads, D), generator=g, device=device,
                    dtype=torch.float32).to(qdt)
    k_scale = v_scale = None
    if w.kv_dtype in ("f32", "bf16", "f16"):
        kdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.kv_dtype]
        kv = torch.randn((npg, 2, P, Hkv, D), generator=g, device=device, dtype=kdt)
    elif w.kv_dtype == "e4m3":
        kv = torch.empty((npg, 2, P, Hkv, D), device=device, dtype=torch.uint8)
        per_token = w.kv_scale == "token"
        sshape = (npg, 2, Hkv, P) if per_token else (npg, 2, Hkv)
        scale = torch.empty(sshape, device=device, dtype=torch.float32)
        for p0 in range(0, npg, chunk_pages):
            p1 = min(npg, p0 + chunk_pages)
            x = torch.randn((p1 - p0, 2, P, Hkv, D), generator=g, device=device,
                            dtype=torch.float32)
            if per_token:
                amax = x.abs().amax(dim=4)  # [pages, 2, P, Hkv]
                s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
                y = (x / s[..., None]).clamp_(-E4M3_MAX, E4M3_MAX)
                s = s.transpose(2, 3)  # [pages, 2, Hkv, P]
            else:
                amax = x.abs().amax(dim=(2, 4))
                s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
                y = (x / s[:, :, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
            kv[p0:p1] = y.to(torch.float8_e4m3fn).view(torch.uint8)
            scale[p0:p1] = s
            del x, y
        k_scale = scale[:, 0].contiguous()
        v_scale = scale[:, 1].contiguous()
    elif w.kv_dtype == "e2m1":
        m = torch.exp(0.5 * torch.randn((2, Hkv, D), generator=g, device=device,
                                        dtype=torch.float32))
        scale = m / 2
        k_scale, v_scale = scale[0].contiguous(), scale[1].contiguous()
        kv = torch.empty((npg, 2, P, Hkv, D // 2), device=device, dtype=torch.uint8)
        for p0 in range(0, npg, chunk_pages):
            p1 = min(npg, p0 + chunk_pages)
            y = 2 * torch.randn((p1 - p0, 2, P, Hkv, D), generator=g, device=device,
                                dtype=torch.float32)
            a = y.abs()
            idx = torch.zeros(y.shape, device=device, dtype=torch.uint8)
            for b, inclusive in E2M1_BOUNDS:
                idx += (a >= b if inclusive else a > b).to(torch.uint8)
            codes = idx | (torch.signbit(y).to(torch.uint8) << 3)
            kv[p0:p1] = codes[..., 0::2] | (codes[..., 1::2] << 4)
            del y, a, idx, codes
    elif w.kv_dtype == "i4":
        m = torch.exp(0.5 * torch.randn((2, Hkv, D), generator=g, device=device,
                                        dtype=torch.float32))
        scale = m / I4_STEPS_PER_SIGMA
        k_scale, v_scale = scale[0].contiguous(), scale[1].contiguous()
        kv = torch.empty((npg, 2, P, Hkv, D // 2), device=device, dtype=torch.uint8)
        for p0 in range(0, npg, chunk_pages):
            p1 = min(npg, p0 + chunk_pages)
            y = torch.randn((p1 - p0, 2, P, Hkv, D), generator=g, device=device,
                            dtype=torch.float32)
            codes = torch.round(y * I4_STEPS_PER_SIGMA).clamp_(-8, 7).to(torch.int8)
            codes = codes.view(torch.uint8) & 0xF
            kv[p0:p1] = codes[..., 0::2] | (codes[..., 1::2] << 4)
            del y, codes
    else:
        raise ValueError(w.kv_dtype)
    if poison:
        unread = torch.from_numpy(~read_mask(table, P)).to(device)
        if w.kv_dtype == "e4m3":
            fill = E4M3_NAN_BYTE
        elif w.kv_dtype == "e2m1":
            fill = E2M1_POISON_BYTE
        elif w.kv_dtype == "i4":
            fill = I4_POISON_BYTE
        else:
            fill = float("nan")
        kvv = kv.permute(0, 2, 1, 3, 4)  # [pages, P, 2, Hkv, D] view
        kvv[unread] = fill
    out = dict(table)
    out.update({"q": q, "kv": kv, "k_scale": k_scale, "v_scale": v_scale, "workload": w})
    return out
