"""Host-side argument checks of the Python binding that run before any device
call: a page table shorter than indptr says, and tensors on another device
than the workspace. CPU only (the wrapper is given a host or meta workspace;
nothing reaches the kernels)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_plan_amd as pk
from paged_kv_decode_plan_amd import wrapper as pw


def _wrapper(device="cpu"):
    w = pw.BatchDecodeWithPagedKVCacheWrapper.__new__(pw.BatchDecodeWithPagedKVCacheWrapper)
    w._ws = torch.empty(1 << 20, dtype=torch.uint8, device=device)
    w._plan = None
    w._indices = None
    return w


@pytest.mark.parametrize("indices", [torch.zeros(4, dtype=torch.int32), np.zeros(4, np.int32),
                                     [0, 1, 2, 3]])
def test_plan_rejects_a_short_page_table(indices):
    w = _wrapper()
    with pytest.raises(ValueError, match="indices holds 4 page ids; indptr\\[-1\\] is 5"):
        w.plan([0, 2, 5], indices, [3, 4], 8, 2, 128, 16, q_data_type=torch.bfloat16,
               kv_data_type=torch.bfloat16, slots=64)
    assert w._plan is None


def test_run_rejects_tensors_on_another_device():
    w = _wrapper("meta")
    w._plan = pw.Plan([0, 2, 5], [3, 4], 8, 2, 128, 16, pk._lib.DTYPE_BF16, pk._lib.DTYPE_BF16,
                      pk._lib.DTYPE_BF16, slots=64)
    w._indices = torch.zeros(5, dtype=torch.int32, device="meta")
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16)
    kv = torch.zeros((6, 2, 16, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q is on cpu; the workspace is on meta"):
        w.run(q, kv)
    with pytest.raises(ValueError, match="k is on cpu"):
        w.run(q.to("meta"), kv)
    with pytest.raises(ValueError, match="out is on cpu"):
        w.run(q.to("meta"), kv.to("meta"), out=torch.empty_like(q))
    w.close()


def test_merge_state_checks_shapes_and_devices():
    v = torch.zeros((3, 2, 8))
    s = torch.zeros((3, 2))
    with pytest.raises(ValueError, match="s_out must be"):
        pk.merge_state(v, s, v, s, s_out=torch.zeros((3, 3)))
    with pytest.raises(ValueError, match="v_b is on meta"):
        pk.merge_state(v, s, v.to("meta"), s)
    with pytest.raises(ValueError, match="device tensors"):
        pk.merge_state(v, s, v, s)
