"""ctypes view of libpkdecode.so (the C ABI of include/pkdecode.h).

Argument marshalling only. The library must be built in-tree
(``python -m paged_kv_decode_plan_amd.build``); loading fails loudly
otherwise — there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkdecode.so")

PKD_OK = 0
PKD_ERR_INVALID_ARGUMENT = -1
PKD_ERR_UNSUPPORTED = -2
PKD_ERR_WORKSPACE_TOO_SMALL = -3
PKD_ERR_PLAN_MISMATCH = -4
PKD_ERR_HIP = -5

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_E4M3 = 2
DTYPE_F16 = 3
DTYPE_E2M1 = 4  # FP4 E2M1, two per byte, per-(KV head, channel) fp32 scales
DTYPE_I4 = 5    # two's-complement int4, two per byte, per-(KV head, channel) fp32 scales
ITEM_COLS = 8  # request, page_begin, page_end, kv_len, partial_slot, q_row, q_len, visible
STAGE_DECODE = 1
STAGE_MERGE = 2
STAGE_ALL = 3

_c_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("indptr", _c_i32p),
        ("last_page_len", _c_i32p),
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("slots", ctypes.c_int32),
        ("balance", ctypes.c_int32),
        ("min_chunk_pages", ctypes.c_int32),
        ("device", ctypes.c_int32),
        ("qo_indptr", _c_i32p),
        ("non_causal", ctypes.c_int32),
        ("capacity_items", ctypes.c_int32),
        ("capacity_merge_tasks", ctypes.c_int32),
        ("capacity_partials", ctypes.c_int32),
        ("capacity_qo_len", ctypes.c_int32),
        ("max_wgs_per_cu", ctypes.c_int32),
        ("kv_scale_per_token", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("chunk_pages", ctypes.c_int32),
        ("num_items", ctypes.c_int32),
        ("num_partials", ctypes.c_int32),
        ("num_split_requests", ctypes.c_int32),
        ("slots", ctypes.c_int32),
        ("balance", ctypes.c_int32),
        ("min_chunk_pages", ctypes.c_int32),
        ("total_kv_tokens", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("query_rows", ctypes.c_int32),
        ("queries_per_item", ctypes.c_int32),
        ("max_qo_len", ctypes.c_int32),
        ("num_merge_tasks", ctypes.c_int32),
        ("units_per_item", ctypes.c_int32),
        ("merge_folded", ctypes.c_int32),
        ("slots_per_cu", ctypes.c_int32),
    ]


class RunArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("indices", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("prior_out", ctypes.c_void_p),
        ("prior_lse", ctypes.c_void_p),
    ]


class MergeStatesArgs(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("v_a", ctypes.c_void_p),
        ("s_a", ctypes.c_void_p),
        ("v_b", ctypes.c_void_p),
        ("s_b", ctypes.c_void_p),
        ("v_out", ctypes.c_void_p),
        ("s_out", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
    ]


class PkdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkdecode error {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_decode_plan_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.pkd_last_error.restype = ctypes.c_char_p
    lib.pkd_last_error.argtypes = []
    lib.pkd_version.restype = ctypes.c_int
    lib.pkd_plan_create.argtypes = [ctypes.POINTER(PlanArgs), ctypes.POINTER(ctypes.c_void_p)]
    lib.pkd_plan_create.restype = ctypes.c_int
    lib.pkd_plan_get_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]
    lib.pkd_plan_get_info.restype = ctypes.c_int
    lib.pkd_plan_get_worklist.argtypes = [ctypes.c_void_p, _c_i32p, _c_i32p, _c_i32p]
    lib.pkd_plan_get_worklist.restype = ctypes.c_int
    lib.pkd_plan_upload.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]
    lib.pkd_plan_upload.restype = ctypes.c_int
    lib.pkd_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(RunArgs)]
    lib.pkd_run.restype = ctypes.c_int
    lib.pkd_run_static.argtypes = [ctypes.c_void_p, ctypes.POINTER(RunArgs)]
    lib.pkd_run_static.restype = ctypes.c_int
    lib.pkd_run_stages.argtypes = [ctypes.c_void_p, ctypes.POINTER(RunArgs), ctypes.c_int32]
    lib.pkd_run_stages.restype = ctypes.c_int
    lib.pkd_run_timed.argtypes = [ctypes.c_void_p, ctypes.POINTER(RunArgs), ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.pkd_run_timed.restype = ctypes.c_int
    lib.pkd_check_page_ids.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64)]
    lib.pkd_check_page_ids.restype = ctypes.c_int
    lib.pkd_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.pkd_plan_destroy.restype = None
    lib.pkd_merge_states.argtypes = [ctypes.POINTER(MergeStatesArgs)]
    lib.pkd_merge_states.restype = ctypes.c_int
    lib.pkd_device_slots.argtypes = [ctypes.c_int32] * 6 + [_c_i32p, _c_i32p]
    lib.pkd_device_slots.restype = ctypes.c_int
    lib.pkd_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.pkd_stream_read.restype = ctypes.c_int
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != PKD_OK:
        msg = load().pkd_last_error().decode(errors="replace")
        raise PkdError(rc, msg)
