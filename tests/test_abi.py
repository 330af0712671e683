"""The C-ABI library loads, exports every declared entry point, and reports
errors through status codes (host-side paths only; no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_decode_plan_amd as pk
from paged_kv_decode_plan_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pkdecode.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkd_[a-z_]+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for n in ["pkd_plan_create", "pkd_plan_get_info", "pkd_plan_get_worklist", "pkd_plan_upload",
              "pkd_run", "pkd_plan_destroy", "pkd_last_error", "pkd_version", "pkd_device_slots"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = pk.load()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_library_has_no_torch_dependency():
    """No shared library the C ABI links against is torch's (sonames only:
    the paths ldd prints depend on the environment)."""
    import subprocess
    out = subprocess.run(["ldd", pk.LIB_PATH], capture_output=True, text=True).stdout
    names = [line.split()[0] for line in out.splitlines() if line.strip()]
    assert names and not [n for n in names if "torch" in n or "c10" in n], names


def _args(**kw):
    indptr = np.array(kw.pop("indptr", [0, 3, 5]), np.int32)
    last = np.array(kw.pop("last", [16, 4]), np.int32)
    a = _lib.PlanArgs()
    a.batch = len(last)
    a.indptr = indptr.ctypes.data_as(_lib._c_i32p)
    a.last_page_len = last.ctypes.data_as(_lib._c_i32p)
    a.num_qo_heads, a.num_kv_heads, a.head_dim, a.page_size = 8, 2, 128, 16
    a.q_dtype = a.kv_dtype = _lib.DTYPE_BF16
    a.out_dtype = _lib.DTYPE_F32
    a.slots = 64
    for k, v in kw.items():
        setattr(a, k, v)
    return a, (indptr, last)


def _create(**kw):
    lib = pk.load()
    a, keep = _args(**kw)
    h = ctypes.c_void_p()
    rc = lib.pkd_plan_create(ctypes.byref(a), ctypes.byref(h))
    return rc, h, lib.pkd_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(indptr=[0, 3, 3], last=[16, 4]), _lib.PKD_ERR_INVALID_ARGUMENT),   # empty request
    (dict(indptr=[0], last=[]), _lib.PKD_ERR_INVALID_ARGUMENT),              # empty batch
    (dict(indptr=[0, 3, 2], last=[16, 4]), _lib.PKD_ERR_INVALID_ARGUMENT),   # decreasing indptr
    (dict(indptr=[1, 3, 5], last=[16, 4]), _lib.PKD_ERR_INVALID_ARGUMENT),   # indptr[0] != 0
    (dict(last=[0, 4]), _lib.PKD_ERR_INVALID_ARGUMENT),
    (dict(last=[17, 4]), _lib.PKD_ERR_INVALID_ARGUMENT),
    (dict(num_qo_heads=7), _lib.PKD_ERR_INVALID_ARGUMENT),                   # Hq % Hkv
    (dict(head_dim=96), _lib.PKD_ERR_UNSUPPORTED),
    (dict(num_qo_heads=128), _lib.PKD_ERR_UNSUPPORTED),                      # group 64
    (dict(num_qo_heads=32, q_dtype=_lib.DTYPE_F32), _lib.PKD_ERR_UNSUPPORTED),  # group 16, fp32 q
    (dict(page_size=12), _lib.PKD_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), _lib.PKD_ERR_UNSUPPORTED),
    (dict(kv_dtype=_lib.DTYPE_I4, q_dtype=_lib.DTYPE_F32), _lib.PKD_ERR_UNSUPPORTED),  # int4: bf16 q
    (dict(kv_dtype=_lib.DTYPE_I4, head_dim=64), _lib.PKD_ERR_UNSUPPORTED),             # int4: D 128
    (dict(q_dtype=_lib.DTYPE_E4M3), _lib.PKD_ERR_UNSUPPORTED),
    (dict(out_dtype=_lib.DTYPE_E4M3), _lib.PKD_ERR_UNSUPPORTED),
    (dict(sm_scale=-1.0), _lib.PKD_ERR_INVALID_ARGUMENT),
    (dict(balance=-1), _lib.PKD_ERR_INVALID_ARGUMENT),
])
def test_plan_create_rejects(kw, code):
    rc, h, msg = _create(**kw)
    assert rc == code, msg
    assert msg and not h.value


def test_plan_create_null_arguments():
    lib = pk.load()
    h = ctypes.c_void_p()
    assert lib.pkd_plan_create(None, ctypes.byref(h)) == _lib.PKD_ERR_INVALID_ARGUMENT
    a, keep = _args()
    a.indptr = ctypes.cast(None, _lib._c_i32p)
    assert lib.pkd_plan_create(ctypes.byref(a), ctypes.byref(h)) == _lib.PKD_ERR_INVALID_ARGUMENT


def test_run_rejects_before_any_device_work():
    lib = pk.load()
    rc, h, msg = _create()
    assert rc == 0, msg
    r = _lib.RunArgs()
    # null pointers
    assert lib.pkd_run(h, ctypes.byref(r)) == _lib.PKD_ERR_INVALID_ARGUMENT
    # non-null but never uploaded: plan mismatch
    fake = 1 << 20
    r.q = r.k = r.v = r.indices = r.out = r.workspace = fake
    r.workspace_bytes = 1 << 30
    assert lib.pkd_run(h, ctypes.byref(r)) == _lib.PKD_ERR_PLAN_MISMATCH
    assert b"workspace" in lib.pkd_last_error()
    lib.pkd_plan_destroy(h)
    lib.pkd_plan_destroy(None)


def test_run_rejects_pages_of_4_gib_or_more():
    """Tile addresses are 32-bit byte offsets within a page on top of the
    page's base, so a page stride of 4 GiB or more is refused up front."""
    lib = pk.load()
    rc, h, msg = _create()
    assert rc == 0, msg
    r = _lib.RunArgs()
    fake = 1 << 20
    r.q = r.k = r.v = r.indices = r.out = r.workspace = fake
    r.workspace_bytes = 1 << 30
    r.token_stride, r.head_stride = 2 * 128, 128
    r.page_stride = (1 << 32) // 2  # bf16: exactly 4 GiB
    assert lib.pkd_run(h, ctypes.byref(r)) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert b"4 GiB" in lib.pkd_last_error()
    r.page_stride = (1 << 32) // 2 - 8  # just under: the plan check comes next
    assert lib.pkd_run(h, ctypes.byref(r)) == _lib.PKD_ERR_PLAN_MISMATCH
    lib.pkd_plan_destroy(h)


def test_upload_rejects_small_or_misaligned_workspace():
    lib = pk.load()
    rc, h, msg = _create()
    assert rc == 0
    info = _lib.PlanInfo()
    assert lib.pkd_plan_get_info(h, ctypes.byref(info)) == 0
    assert lib.pkd_plan_upload(h, ctypes.c_void_p(1 << 20), info.workspace_bytes - 1,
                               None) == _lib.PKD_ERR_WORKSPACE_TOO_SMALL
    assert lib.pkd_plan_upload(h, ctypes.c_void_p((1 << 20) + 16), info.workspace_bytes,
                               None) == _lib.PKD_ERR_INVALID_ARGUMENT
    lib.pkd_plan_destroy(h)


def test_error_message_is_thread_local():
    import threading
    lib = pk.load()
    _create(last=[0, 4])
    main_msg = lib.pkd_last_error()
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.pkd_last_error()))
    t.start()
    t.join()
    assert main_msg and seen == [b""]


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_check_page_ids_rejects_bad_arguments():
    lib = pk.load()
    cnt = ctypes.c_int64()
    assert lib.pkd_check_page_ids(None, 4, 8, None, None, None) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_check_page_ids(None, -1, 8, None, ctypes.byref(cnt), None) == \
        _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_check_page_ids(None, 4, -1, None, ctypes.byref(cnt), None) == \
        _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_check_page_ids(None, 4, 8, None, ctypes.byref(cnt), None) == \
        _lib.PKD_ERR_INVALID_ARGUMENT  # null indices with a positive count


def test_stream_read_rejects_bad_arguments():
    """The calibration read checks its arguments on the host before launching."""
    lib = pk.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.pkd_stream_read(None, 1 << 20, 256, fake, None) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_stream_read(fake, 1 << 20, 256, None, None) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_stream_read(ctypes.c_void_p(0x1008), 1 << 20, 256, fake,
                               None) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_stream_read(fake, 100, 256, fake, None) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert lib.pkd_stream_read(fake, 1 << 20, 0, fake, None) == _lib.PKD_ERR_INVALID_ARGUMENT
    assert b"workgroups" in lib.pkd_last_error()


def test_static_scratch_run_refuses_large_plans_before_device_work():
    """pkd_run_static checks its arguments and the plan's scratch need (16 MiB
    at most) on the host before any HIP call."""
    lib = pk.load()
    indptr = list(range(0, 65 * 128, 128))
    rc, h, msg = _create(indptr=indptr, last=[16] * 64, num_qo_heads=32, num_kv_heads=8,
                         slots=16384, balance=1, min_chunk_pages=1)
    assert rc == 0, msg
    info = _lib.PlanInfo()
    assert lib.pkd_plan_get_info(h, ctypes.byref(info)) == 0
    assert info.workspace_bytes > 16 << 20
    r = _lib.RunArgs()
    assert lib.pkd_run_static(h, ctypes.byref(r)) == _lib.PKD_ERR_INVALID_ARGUMENT
    fake = 1 << 20
    r.q = r.k = r.v = r.indices = r.out = fake  # never dereferenced: refused first
    assert lib.pkd_run_static(h, ctypes.byref(r)) == _lib.PKD_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.pkd_last_error()
    assert lib.pkd_run_static(None, ctypes.byref(r)) == _lib.PKD_ERR_INVALID_ARGUMENT
    lib.pkd_plan_destroy(h)
