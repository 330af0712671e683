"""Python binding with the plan()/run() shape of the paged-KV decode wrapper.

"FlashDecoding + FlashInfer — the decode-time attention story", §"The API you
actually use (Python)": a wrapper owns a caller-allocated workspace and a KV
layout ("NHD"); plan() takes the page table (indptr, indices, last_page_len),
head counts, head_dim, page_size and dtypes once per batch shape; run(q,
paged_kv_cache) is the hot path. The quick-start of "GitHub Spotlight:
FlashInfer" calls the same two steps begin_forward()/forward(); both names
are accepted.

Everything here is argument marshalling for libpkdecode.so; PyTorch supplies
device memory and the current stream only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import numpy as np

from . import _lib

DEFAULT_WORKSPACE_BYTES = 128 * 1024 * 1024


def _dtype_code(dt) -> int:
    import torch
    if dt in (torch.float32, "f32", "float32"):
        return _lib.DTYPE_F32
    if dt in (torch.bfloat16, "bf16", "bfloat16"):
        return _lib.DTYPE_BF16
    if dt in (torch.float8_e4m3fn, torch.uint8, "e4m3", "float8_e4m3fn"):
        return _lib.DTYPE_E4M3
    if dt in (torch.float16, "f16", "float16"):
        return _lib.DTYPE_F16
    if dt in (getattr(torch, "float4_e2m1fn_x2", "e2m1"), "e2m1", "float4_e2m1fn_x2"):
        return _lib.DTYPE_E2M1
    if dt in ("i4", "int4"):
        return _lib.DTYPE_I4
    raise ValueError(f"unsupported dtype {dt}")


def _host_i32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


class Plan:
    """A plan handle (host partition + workspace layout). Host-only until uploaded."""

    def __init__(self, indptr, last_page_len, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, page_size: int, q_dtype: int, kv_dtype: int, out_dtype: int,
                 sm_scale: Optional[float] = None, slots: int = 0, balance: int = 0,
                 min_chunk_pages: int = 0, device: int = 0, qo_indptr=None,
                 causal: bool = True, capacity=None, max_wgs_per_cu: int = 0,
                 kv_scale: str = "page"):
        lib = _lib.load()
        self._lib = lib
        self._handle = ctypes.c_void_p()
        self.indptr = _host_i32(indptr)
        self.last_page_len = _host_i32(last_page_len)
        B = len(self.last_page_len)
        if len(self.indptr) != B + 1:
            raise ValueError("indptr must have batch+1 entries")
        self.qo_indptr = None if qo_indptr is None else _host_i32(qo_indptr)
        if self.qo_indptr is not None and len(self.qo_indptr) != B + 1:
            raise ValueError("qo_indptr must have batch+1 entries")
        a = _lib.PlanArgs()
        a.batch = B
        a.indptr = self.indptr.ctypes.data_as(_lib._c_i32p)
        a.last_page_len = self.last_page_len.ctypes.data_as(_lib._c_i32p)
        a.num_qo_heads = num_qo_heads
        a.num_kv_heads = num_kv_heads
        a.head_dim = head_dim
        a.page_size = page_size
        a.q_dtype = q_dtype
        a.kv_dtype = kv_dtype
        a.out_dtype = out_dtype
        a.sm_scale = 0.0 if sm_scale is None else float(sm_scale)
        a.slots = slots
        a.balance = balance
        a.min_chunk_pages = min_chunk_pages
        a.device = device
        if self.qo_indptr is not None:
            a.qo_indptr = self.qo_indptr.ctypes.data_as(_lib._c_i32p)
        a.non_causal = 0 if causal else 1
        a.max_wgs_per_cu = max_wgs_per_cu
        if kv_scale not in ("page", "token"):
            raise ValueError("kv_scale must be 'page' or 'token'")
        a.kv_scale_per_token = 1 if kv_scale == "token" else 0
        self.kv_scale = kv_scale
        if capacity is not None:
            c = _capacity(capacity)
            (a.capacity_items, a.capacity_merge_tasks, a.capacity_partials,
             a.capacity_qo_len) = c
        _lib.check(lib.pkd_plan_create(ctypes.byref(a), ctypes.byref(self._handle)))
        info = _lib.PlanInfo()
        _lib.check(lib.pkd_plan_get_info(self._handle, ctypes.byref(info)))
        self.info = {f: getattr(info, f) for f, _ in _lib.PlanInfo._fields_}
        self.batch, self.num_qo_heads, self.num_kv_heads = B, num_qo_heads, num_kv_heads
        self.query_rows = self.info["query_rows"]
        self.head_dim, self.page_size = head_dim, page_size
        self.q_dtype, self.kv_dtype, self.out_dtype = q_dtype, kv_dtype, out_dtype

    def worklist(self):
        """(items int32[num_items, 8], merge_indptr int32[B+1], split_requests int32[S])."""
        n = self.info["num_items"]
        items = np.zeros((n, _lib.ITEM_COLS), dtype=np.int32)
        merge = np.zeros(self.batch + 1, dtype=np.int32)
        split = np.zeros(max(1, self.info["num_split_requests"]), dtype=np.int32)
        _lib.check(self._lib.pkd_plan_get_worklist(
            self._handle, items.ctypes.data_as(_lib._c_i32p), merge.ctypes.data_as(_lib._c_i32p),
            split.ctypes.data_as(_lib._c_i32p)))
        return items, merge, split[: self.info["num_split_requests"]]

    def upload(self, workspace_ptr: int, workspace_bytes: int, stream_ptr: int) -> None:
        _lib.check(self._lib.pkd_plan_upload(self._handle, ctypes.c_void_p(workspace_ptr),
                                             ctypes.c_size_t(workspace_bytes),
                                             ctypes.c_void_p(stream_ptr)))

    def run_raw(self, args: "_lib.RunArgs", stages: int = _lib.STAGE_ALL, events=None,
                static_scratch: bool = False) -> None:
        if static_scratch:  # the library's static device scratch, no workspace
            if stages != _lib.STAGE_ALL or events is not None:
                raise ValueError("the static-scratch run takes whole runs without events")
            _lib.check(self._lib.pkd_run_static(self._handle, ctypes.byref(args)))
        elif events is not None:  # raw hipEvent_t handles stamped by the decode kernel's dispatch
            _lib.check(self._lib.pkd_run_timed(self._handle, ctypes.byref(args), stages,
                                               ctypes.c_void_p(events[0]),
                                               ctypes.c_void_p(events[1])))
        elif stages == _lib.STAGE_ALL:
            _lib.check(self._lib.pkd_run(self._handle, ctypes.byref(args)))
        else:
            _lib.check(self._lib.pkd_run_stages(self._handle, ctypes.byref(args), stages))

    def close(self) -> None:
        if getattr(self, "_handle", None) and self._handle.value:
            self._lib.pkd_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _capacity(capacity) -> Tuple[int, int, int, int]:
    """(items, merge_tasks, partials, qo_len) from a dict with those keys or a tuple."""
    if isinstance(capacity, dict):
        return (int(capacity["items"]), int(capacity["merge_tasks"]),
                int(capacity["partials"]), int(capacity.get("qo_len", 1)))
    items, tasks, parts, *rest = capacity
    return int(items), int(tasks), int(parts), int(rest[0]) if rest else 1


def plan_partition(indptr, last_page_len, num_qo_heads, num_kv_heads, head_dim, page_size,
                   kv_dtype="bf16", q_dtype="bf16", out_dtype="f32", slots=1024, balance=0,
                   min_chunk_pages=0, qo_indptr=None, causal=True, capacity=None,
                   kv_scale="page"):
    """Build a plan and return its decisions (info, work list, merge index,
    split requests). Host-only with an explicit slot count; ``slots=0`` asks
    the device (device 0) for its resident-workgroup count, as run()'s
    default plans do."""
    p = Plan(indptr, last_page_len, num_qo_heads, num_kv_heads, head_dim, page_size,
             _dtype_code(q_dtype), _dtype_code(kv_dtype), _dtype_code(out_dtype), None, slots,
             balance, min_chunk_pages, qo_indptr=qo_indptr, causal=causal, capacity=capacity,
             kv_scale=kv_scale)
    items, merge, split = p.worklist()
    info = dict(p.info)
    p.close()
    return info, items, merge, split


def _same_device(device, **tensors):
    """Every tensor given (None skipped) must live on `device`: the kernels take
    raw pointers, and one on another device (or in host memory) would be read
    as if it were on this one."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}; the workspace is on {device}")


def _split_kv(paged_kv_cache):
    """(k, v) views from a combined [pages, 2, P, Hkv, D] tensor or a (k, v) pair."""
    if isinstance(paged_kv_cache, (tuple, list)):
        k, v = paged_kv_cache
    else:
        if paged_kv_cache.dim() != 5 or paged_kv_cache.shape[1] != 2:
            raise ValueError("combined NHD cache must be [num_pages, 2, page_size, Hkv, head_dim]")
        k, v = paged_kv_cache[:, 0], paged_kv_cache[:, 1]
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("K and V pools must have the same shape and strides")
    if k.dim() != 4 or k.stride(3) != 1:
        raise ValueError("K/V pools must be [num_pages, page_size, Hkv, head_dim] with head_dim contiguous")
    return k, v


class BatchDecodeWithPagedKVCacheWrapper:
    """plan()/run() wrapper over libpkdecode for one device and one workspace."""

    def __init__(self, workspace_buffer, kv_layout: str = "NHD"):
        if kv_layout != "NHD":
            raise ValueError("only the NHD layout is supported")
        if not workspace_buffer.is_cuda:
            raise ValueError("the workspace must be device memory")
        self._ws = workspace_buffer
        self._plan: Optional[Plan] = None
        self._indices = None

    # -- plan ----------------------------------------------------------------
    def plan(self, indptr, indices, last_page_len, num_qo_heads: int, num_kv_heads: int,
             head_dim: int, page_size: int, pos_encoding_mode: str = "NONE",
             q_data_type=None, kv_data_type=None, out_data_type=None, data_type=None,
             sm_scale: Optional[float] = None, slots: int = 0, balance: int = 0,
             min_chunk_pages: int = 0, qo_indptr=None, causal: bool = True,
             capacity=None, max_wgs_per_cu: int = 0, kv_scale: str = "page") -> None:
        """Plan one batch. ``qo_indptr`` (host, [batch+1]) gives request r the q
        rows ``qo_indptr[r]:qo_indptr[r+1]``: its newest tokens, attended
        causally; omitted, every request has one query token (q row r). With
        ``causal=False`` every row sees all of its request's tokens (the
        shared-prefix level of cascade attention). ``capacity`` (dict with
        ``items``, ``merge_tasks``, ``partials``, ``qo_len``) makes a
        fixed-capacity plan: run() then launches the same grids with the same
        arguments for every such plan, so a captured HIP graph of run() stays
        valid across plan()/upload of new batches. ``kv_scale`` (e4m3 KV):
        ``"page"`` for one scale per (page, KV head), ``"token"`` for one per
        (token, KV head). FP4 E2M1 KV (``kv_data_type`` "e2m1" or
        ``torch.float4_e2m1fn_x2``) is a byte pool ``[..., head_dim // 2]``
        (uint8 or float4_e2m1fn_x2, element 2i in the low nibble of byte i)
        with scales ``[num_kv_heads, head_dim]`` per channel; int4 KV
        (``kv_data_type`` "i4" or "int4": two's-complement codes -8 .. 7,
        value = code x scale) is a uint8 pool of the same layout."""
        import torch
        if pos_encoding_mode != "NONE":
            raise ValueError("only pos_encoding_mode='NONE' is supported")
        q_dt = q_data_type or data_type or torch.bfloat16
        kv_dt = kv_data_type or data_type or q_dt
        out_dt = out_data_type or q_dt
        host_indptr = _host_i32(indptr)
        n_indices = (indices.numel() if isinstance(indices, torch.Tensor)
                     else int(np.asarray(indices).size))
        if len(host_indptr) and n_indices < int(host_indptr[-1]):
            # the kernels read page ids indices[indptr[r] .. indptr[r+1]) on the
            # device; a shorter table would be read past its end
            raise ValueError(f"indices holds {n_indices} page ids; indptr[-1] is "
                             f"{int(host_indptr[-1])}")
        if self._plan is not None:
            self._plan.close()
            self._plan = None
        dev = self._ws.device.index or 0
        indptr = host_indptr
        self._plan = Plan(indptr, last_page_len, num_qo_heads, num_kv_heads, head_dim, page_size,
                          _dtype_code(q_dt), _dtype_code(kv_dt), _dtype_code(out_dt), sm_scale,
                          slots, balance, min_chunk_pages, dev, qo_indptr=qo_indptr,
                          causal=causal, capacity=capacity, max_wgs_per_cu=max_wgs_per_cu,
                          kv_scale=kv_scale)
        self._indices = indices if isinstance(indices, torch.Tensor) else torch.as_tensor(
            np.asarray(indices, dtype=np.int32))
        if self._indices.device != self._ws.device or self._indices.dtype != torch.int32:
            self._indices = self._indices.to(device=self._ws.device, dtype=torch.int32)
        self._indices = self._indices.contiguous()
        need = self._plan.info["workspace_bytes"]
        have = self._ws.numel() * self._ws.element_size()
        if have < need:
            raise _lib.PkdError(_lib.PKD_ERR_WORKSPACE_TOO_SMALL,
                                f"workspace has {have} bytes, the plan needs {need}")
        stream = torch.cuda.current_stream(self._ws.device).cuda_stream
        self._plan.upload(self._ws.data_ptr(), have, stream)

    begin_forward = plan

    @property
    def plan_info(self) -> dict:
        return dict(self._plan.info)

    # -- run -----------------------------------------------------------------
    def run(self, q, paged_kv_cache, out=None, lse=None, return_lse: bool = False,
            k_scale=None, v_scale=None, stages: int = _lib.STAGE_ALL, decode_events=None,
            check_page_ids: bool = False, prior=None, static_scratch: bool = False):
        """``decode_events``: an optional pair of ``torch.cuda.Event(enable_timing=True)``
        that the decode kernel's own dispatch records as it starts and completes
        (``pkd_run_timed``); ``start.elapsed_time(stop)`` is then the kernel's time.
        ``check_page_ids`` (or ``PKD_DEBUG_CHECKS=1`` in the environment): before
        launching, count the plan's page ids outside the pool
        (``pkd_check_page_ids``, which synchronises the stream) and raise
        ``PkdError`` (INVALID_ARGUMENT) instead of running on such a table.
        ``prior``: ``(v, lse)``, another normalised result of the same rows over a
        disjoint token set (float32 ``[rows, Hq, head_dim]`` and ``[rows, Hq]``),
        merged into the output as it is written (cascade attention's levels).
        ``static_scratch``: run through ``pkd_run_static``, which keeps the
        plan's work list and partial states in the library's own device scratch
        instead of the workspace (for callers that cannot allocate; the binding
        itself still allocates ``out``/``lse`` when they are not given)."""
        import torch
        p = self._plan
        if p is None:
            raise RuntimeError("plan() must be called before run()")
        k, v = _split_kv(paged_kv_cache)
        _same_device(self._ws.device, q=q, k=k, v=v, out=out, lse=lse, k_scale=k_scale,
                     v_scale=v_scale, prior_v=None if prior is None else prior[0],
                     prior_lse=None if prior is None else prior[1])
        if q.shape != (p.query_rows, p.num_qo_heads, p.head_dim) or not q.is_contiguous():
            raise ValueError(
                f"q must be contiguous [{p.query_rows}, {p.num_qo_heads}, {p.head_dim}]")
        fp4 = p.kv_dtype in (_lib.DTYPE_E2M1, _lib.DTYPE_I4)  # 4-bit codes, two per byte
        kv_ok = (k.dtype in (torch.uint8, getattr(torch, "float4_e2m1fn_x2", torch.uint8)) if fp4
                 else _dtype_code(k.dtype) == p.kv_dtype)
        if _dtype_code(q.dtype) != p.q_dtype or not kv_ok:
            raise _lib.PkdError(_lib.PKD_ERR_PLAN_MISMATCH, "q/KV dtypes differ from the plan")
        row = p.head_dim // 2 if fp4 else p.head_dim  # storage units per row
        if k.shape[1] != p.page_size or k.shape[2] != p.num_kv_heads or k.shape[3] != row:
            raise ValueError("KV pool shape disagrees with the plan")
        out_dt = {_lib.DTYPE_F32: torch.float32, _lib.DTYPE_BF16: torch.bfloat16,
                  _lib.DTYPE_F16: torch.float16}[p.out_dtype]
        if out is None:
            out = torch.empty(q.shape, dtype=out_dt, device=q.device)
        elif out.dtype != out_dt or out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out has the wrong dtype, shape or layout")
        if return_lse and lse is None:
            lse = torch.empty((p.query_rows, p.num_qo_heads), dtype=torch.float32, device=q.device)
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise ValueError("lse must be contiguous float32 [batch, num_qo_heads]")
        a = _lib.RunArgs()
        a.q = q.data_ptr()
        a.k = k.data_ptr()
        a.v = v.data_ptr()
        per = 2 if fp4 else 1  # strides in elements: two 4-bit codes per byte
        a.page_stride, a.token_stride, a.head_stride = (per * k.stride(0), per * k.stride(1),
                                                        per * k.stride(2))
        a.indices = self._indices.data_ptr()
        if p.kv_dtype == _lib.DTYPE_E4M3:
            if k_scale is None or v_scale is None:
                raise ValueError("e4m3 KV needs k_scale and v_scale [num_pages, num_kv_heads]")
            want = ((k.shape[0], p.num_kv_heads, p.page_size) if p.kv_scale == "token"
                    else (k.shape[0], p.num_kv_heads))
            for s in (k_scale, v_scale):
                if s.dtype != torch.float32 or not s.is_contiguous() or tuple(s.shape) != want:
                    raise ValueError(f"scales must be contiguous float32 {list(want)}")
            a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
        elif fp4:
            want = (p.num_kv_heads, p.head_dim)
            if k_scale is None or v_scale is None:
                raise ValueError(f"4-bit KV needs k_scale and v_scale {list(want)}")
            for s in (k_scale, v_scale):
                if s.dtype != torch.float32 or not s.is_contiguous() or tuple(s.shape) != want:
                    raise ValueError(f"scales must be contiguous float32 {list(want)}")
            a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
        a.out = out.data_ptr()
        a.lse = lse.data_ptr() if lse is not None else None
        if prior is not None:
            pv, pl = prior
            if (pv.dtype != torch.float32 or pl.dtype != torch.float32 or pv.shape != q.shape
                    or tuple(pl.shape) != (p.query_rows, p.num_qo_heads)
                    or not (pv.is_contiguous() and pl.is_contiguous())):
                raise ValueError("prior must be contiguous float32 ([rows, Hq, D], [rows, Hq])")
            a.prior_out, a.prior_lse = pv.data_ptr(), pl.data_ptr()
        a.workspace = self._ws.data_ptr()
        a.workspace_bytes = self._ws.numel() * self._ws.element_size()
        a.stream = torch.cuda.current_stream(q.device).cuda_stream
        if check_page_ids or os.environ.get("PKD_DEBUG_CHECKS") == "1":
            bad, first = ctypes.c_int64(), ctypes.c_int64()
            _lib.check(_lib.load().pkd_check_page_ids(
                ctypes.c_void_p(self._indices.data_ptr()), ctypes.c_int64(self._indices.numel()),
                ctypes.c_int32(k.shape[0]), ctypes.c_void_p(a.stream), ctypes.byref(bad),
                ctypes.byref(first)))
            if bad.value:
                raise _lib.PkdError(
                    _lib.PKD_ERR_INVALID_ARGUMENT,
                    f"{bad.value} page ids lie outside the pool of {k.shape[0]} pages "
                    f"(the first at position {first.value} of indices)")
        events = None
        if decode_events is not None:
            for ev in decode_events:
                if not ev.cuda_event:  # torch creates the HIP event at its first record
                    ev.record()
            events = (decode_events[0].cuda_event, decode_events[1].cuda_event)
        p.run_raw(a, stages, events, static_scratch=static_scratch)
        return (out, lse) if (return_lse or lse is not None) else out

    forward = run

    def close(self) -> None:
        if self._plan is not None:
            self._plan.close()
            self._plan = None


def merge_state(v_a, s_a, v_b, s_b, v_out=None, s_out=None, out_dtype=None):
    """Merge two normalised attention results of the same rows over disjoint
    token sets (``v`` [rows, heads, head_dim] float32/bfloat16, ``s`` float32
    [rows, heads] natural-log LSE; -inf marks an empty side). Returns
    ``(v_out, s_out)``; runs ``pkd_merge_states`` on the current stream."""
    import torch
    if v_a.shape != v_b.shape or v_a.dtype != v_b.dtype or v_a.dim() != 3:
        raise ValueError("v_a and v_b must be [rows, heads, head_dim] of one dtype")
    for s in (s_a, s_b):
        if s.shape != v_a.shape[:2] or s.dtype != torch.float32 or not s.is_contiguous():
            raise ValueError("s_a and s_b must be contiguous float32 [rows, heads]")
    if not (v_a.is_contiguous() and v_b.is_contiguous()):
        raise ValueError("v_a and v_b must be contiguous")
    odt = out_dtype or (v_out.dtype if v_out is not None else v_a.dtype)
    if v_out is None:
        v_out = torch.empty(v_a.shape, dtype=odt, device=v_a.device)
    elif v_out.shape != v_a.shape or v_out.dtype != odt or not v_out.is_contiguous():
        raise ValueError("v_out has the wrong shape, dtype or layout")
    if s_out is None:
        s_out = torch.empty(v_a.shape[:2], dtype=torch.float32, device=v_a.device)
    elif s_out.shape != v_a.shape[:2] or s_out.dtype != torch.float32 or not s_out.is_contiguous():
        raise ValueError("s_out must be contiguous float32 [rows, heads]")
    _same_device(v_a.device, v_b=v_b, s_a=s_a, s_b=s_b, v_out=v_out, s_out=s_out)
    if not v_a.is_cuda:
        raise ValueError("merge_state works on device tensors")
    a = _lib.MergeStatesArgs()
    a.rows, a.num_heads, a.head_dim = v_a.shape
    a.in_dtype = _dtype_code(v_a.dtype)
    a.out_dtype = _dtype_code(odt)
    a.v_a, a.s_a, a.v_b, a.s_b = v_a.data_ptr(), s_a.data_ptr(), v_b.data_ptr(), s_b.data_ptr()
    a.v_out, a.s_out = v_out.data_ptr(), s_out.data_ptr()
    a.stream = torch.cuda.current_stream(v_a.device).cuda_stream
    _lib.check(_lib.load().pkd_merge_states(ctypes.byref(a)))
    return v_out, s_out


class CascadeBatchDecodeWrapper:
    """Two-level cascade decode: the queries of all requests that share a
    prefix attend to it once, as one non-causal request of the plan (level
    0); each request attends to its own suffix pages (level 1), and level 1
    merges level 0's normalised result into its rows as it writes them (the
    rule of ``merge_state``, without a separate launch).

    Requests must be ordered by prefix group: group p owns the q rows
    ``shared_qo_indptr[p]:shared_qo_indptr[p+1]`` (one per request). The
    caller's workspace is split in two halves, one per level.
    """

    def __init__(self, workspace_buffer, kv_layout: str = "NHD"):
        half = (workspace_buffer.numel() * workspace_buffer.element_size() // 2) // 256 * 256
        raw = workspace_buffer.view(-1).view(__import__("torch").uint8)
        self._levels = (BatchDecodeWithPagedKVCacheWrapper(raw[:half], kv_layout),
                        BatchDecodeWithPagedKVCacheWrapper(raw[half:2 * half], kv_layout))
        self._rows = 0

    def plan(self, shared_indptr, shared_indices, shared_last_page_len, shared_qo_indptr,
             unique_indptr, unique_indices, unique_last_page_len, num_qo_heads: int,
             num_kv_heads: int, head_dim: int, page_size: int, q_data_type=None,
             kv_data_type=None, out_data_type=None, sm_scale: Optional[float] = None,
             slots: int = 0, balance: int = 0, min_chunk_pages: int = 0) -> None:
        import torch
        qo = _host_i32(shared_qo_indptr)
        rows = len(_host_i32(unique_last_page_len))
        if int(qo[-1]) != rows:
            raise ValueError("the prefix groups must cover every request exactly once")
        kw = dict(q_data_type=q_data_type, kv_data_type=kv_data_type,
                  out_data_type=torch.float32, sm_scale=sm_scale, slots=slots,
                  balance=balance, min_chunk_pages=min_chunk_pages)
        self._levels[0].plan(shared_indptr, shared_indices, shared_last_page_len, num_qo_heads,
                             num_kv_heads, head_dim, page_size, qo_indptr=qo, causal=False, **kw)
        self._out_dtype = out_data_type or q_data_type or torch.bfloat16
        kw["out_data_type"] = self._out_dtype  # the second level writes the merged rows
        self._levels[1].plan(unique_indptr, unique_indices, unique_last_page_len, num_qo_heads,
                             num_kv_heads, head_dim, page_size, **kw)
        self._rows, self._heads, self._dim = rows, num_qo_heads, head_dim

    def run(self, q, paged_kv_cache, out=None, return_lse: bool = False, k_scale=None,
            v_scale=None):
        import torch
        shape = (self._rows, self._heads, self._dim)
        # the shared level in float32, then each request's own pages with the
        # shared result merged in as the output is written
        o = torch.empty(shape, dtype=torch.float32, device=q.device)
        s = torch.empty(shape[:2], dtype=torch.float32, device=q.device)
        self._levels[0].run(q, paged_kv_cache, out=o, lse=s, k_scale=k_scale, v_scale=v_scale)
        if out is None:
            out = torch.empty(shape, dtype=self._out_dtype, device=q.device)
        lse = torch.empty(shape[:2], dtype=torch.float32, device=q.device) if return_lse else None
        self._levels[1].run(q, paged_kv_cache, out=out, lse=lse, k_scale=k_scale, v_scale=v_scale,
                            prior=(o, s))
        return (out, lse) if return_lse else out

    def close(self) -> None:
        for w in self._levels:
            w.close()


def stream_read(buf, workgroups: int, sink=None):
    """Enqueue the calibration read (``pkd_stream_read``) of the whole of the
    contiguous device tensor ``buf`` by ``workgroups`` workgroups on the current
    stream; returns the uint32 sink ``[4 * workgroups]`` it writes."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(4 * workgroups, dtype=torch.int32, device=buf.device)
    elif sink.numel() < 4 * workgroups or sink.element_size() != 4 or sink.device != buf.device:
        raise ValueError("sink must hold 4 * workgroups 32-bit words on buf's device")
    stream = torch.cuda.current_stream(buf.device).cuda_stream
    _lib.check(_lib.load().pkd_stream_read(
        ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(buf.numel() * buf.element_size()),
        ctypes.c_int32(workgroups), ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)))
    return sink
