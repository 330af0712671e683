"""pkd_run_timed: the decode kernel's dispatch records the caller's events;
the work and the result are those of run().

Checked on the GPU: the outputs equal run()'s bit for bit (one-token and
split plans, the merge folded or separate), and the kernel's own interval is
positive and lies inside a bracket of events recorded around the launch.
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_plan_amd as pk
from gpu_helpers import compare, oracle_for, to_device, workspace
from workloads import custom_workload, host_case

pytestmark = pytest.mark.gpu


def _plan(dc, **kw):
    w = dc["workload"]
    wr = pk.BatchDecodeWithPagedKVCacheWrapper(workspace(), "NHD")
    wr.plan(dc["indptr"], dc["indices"], dc["last_page_len"], w.num_qo_heads, w.num_kv_heads,
            w.head_dim, w.page_size, q_data_type=dc["q"].dtype, kv_data_type=dc["kv"].dtype,
            out_data_type=torch.float32, sm_scale=w.scale(), **kw)
    return wr


@pytest.mark.parametrize("split", ["none", "split", "separate"])
def test_timed_run_matches_run_and_stamps_the_kernel(split):
    lens = [2048] * 6 + [37, 900]
    w = custom_workload(len(lens), 32, 8, 128, 16, "bf16", "bf16", lens,
                        pool_pages=sum(-(-x // 16) for x in lens) + 5)
    case = host_case(w, 4242, poison=True)
    print("[gpu] timed run, split", split, flush=True)
    dc = to_device(case)
    kw = {} if split == "none" else dict(slots=64, balance=1, min_chunk_pages=1)
    wr = _plan(dc, **kw)
    info = wr.plan_info
    if split != "none":
        assert info["num_split_requests"] > 0
    stages = pk._lib.STAGE_DECODE if split == "separate" else pk._lib.STAGE_ALL
    ref, ref_lse = wr.run(dc["q"], dc["kv"], return_lse=True)
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    inner = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    out = torch.empty_like(ref)
    lse = torch.empty_like(ref_lse)
    for _ in range(2):  # the second pass reuses events the library has stamped
        outer[0].record()
        wr.run(dc["q"], dc["kv"], out=out, lse=lse, stages=stages, decode_events=inner)
        if split == "separate":
            wr.run(dc["q"], dc["kv"], out=out, lse=lse, stages=pk._lib.STAGE_MERGE)
        outer[1].record()
        torch.cuda.synchronize()
        k_ms = inner[0].elapsed_time(inner[1])
        b_ms = outer[0].elapsed_time(outer[1])
        assert 0.0 < k_ms <= b_ms, (k_ms, b_ms)
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    wr.close()
    ref_out, ref_l = oracle_for(case)
    compare(out, lse, ref_out, ref_l, "bf16")


@pytest.mark.parametrize("workgroups", [1, 256, 1024])
def test_stream_read_reads_every_word(workgroups):
    """The calibration read folds every 32-bit word of the buffer into its sink
    (XOR over all sink words = XOR over the buffer), for a buffer that ends in
    a ragged tail of its last 32 KiB block."""
    rng = np.random.default_rng(workgroups)
    words = rng.integers(-2**31, 2**31, size=(10 << 20) // 4 + 12, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(words).to("cuda:0")
    print("[gpu] stream_read", workgroups, flush=True)
    sink = pk.stream_read(buf, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words.view(np.uint32))
