#!/usr/bin/env python3
"""Benchmark: batched paged-KV decode attention on one MI355X.

One step is one run() over the whole batch: the split-KV decode kernel and,
for a plan that splits requests, the merge of their partial states (folded
into the decode kernel for a few short splits, else the merge kernel). The
default workload is the heterogeneous ragged batch, the largest that the
measurements cover and the one the load balancing is for (B=256, 32 query /
8 KV heads, head_dim 128, 16-token pages, bf16, context lengths log-uniform
in [256, 65536]); ``--config`` selects another. Inputs are synthetic (seeded
normal values, shuffled page table) and resident in HBM before timing.

Timing: W untimed warmup steps, then K timed steps. Before each timed step a
1 GiB buffer is read so that neither L2 nor the 256 MB last-level cache holds
KV; HIP events on the launch stream bracket every step (with
``--separate-merge``, the decode and merge stages apart). ``value`` is KV-read
GB/s over the whole step (algorithmic KV bytes / mean step time).
With ``--layers L`` a step is L run() calls of its one plan, each over its
own copy of the KV pool, and every time is reported per layer (the
dispatch-stamped kernel series is then left out: the bracket is the figure).
``roofline`` is for the decode kernel, timed over K more cold steps by
events that its own dispatch records (hipExtLaunchKernel through
pkd_run_timed); HBM traffic comes from the committed rocprofv3 counter
summary when it was taken on the current kernel sources. ``cpu_baseline``
times the float64 oracle on a bounded sample of the same batch (about 12 s
of work) on one host core (and its ``parallel`` entry, the same sample over
single-threaded worker processes, one per core of this process's affinity
mask up to 16, the CPU share of one GPU on the measurement hosts);
``calibration`` times the library's plain streaming-read kernel
(``pkd_stream_read``) over the 1 GiB flush buffer with 1, 2 and 4
workgroups per compute unit on the same device.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PLAN_KEYS = ("chunk_pages", "num_items", "num_partials", "num_split_requests", "slots",
             "balance", "min_chunk_pages", "queries_per_item")
METRIC = "KV-read HBM GB/s (% of peak) + µs per batched decode step"
CSRC = os.path.join(ROOT, "paged_kv_decode_plan_amd", "csrc")


ELEM_BITS = {"f32": 32, "bf16": 16, "f16": 16, "e4m3": 8, "e2m1": 4, "i4": 4}


def kv_bytes(w, table, logical: bool = False) -> int:
    """Algorithmic bytes the decode kernel must read: every valid K and V element
    once, plus for e4m3 the fp32 K and V scale of every (page, KV head) (or
    token and KV head) and for e2m1 and int4 the fp32 K and V scale of every
    (KV head, channel). With a shared prefix (cascade) each group's prefix counts once,
    unless `logical` (every request's full context, as plain decode would read
    it)."""
    tokens = int(table["kv_lens"].sum())
    if w.shared_prefix is not None and not logical:
        groups, prefix = w.shared_prefix
        tokens = tokens - len(table["kv_lens"]) * prefix + groups * prefix
    b = tokens * w.num_kv_heads * w.head_dim * 2 * ELEM_BITS[w.kv_dtype] // 8
    if w.kv_dtype in ("e2m1", "i4"):
        b += w.num_kv_heads * w.head_dim * 2 * 4
    elif w.kv_dtype == "e4m3" and w.kv_scale == "token":
        b += tokens * w.num_kv_heads * 2 * 4
    elif w.kv_dtype == "e4m3":
        pages = int(table["indptr"][-1])
        b += pages * w.num_kv_heads * 2 * 4
    return b


# The sources the decode kernels are built and launched from: a change to any
# of them makes committed counter readings of the decode kernel stale.
DECODE_SOURCES = ("decode_mfma.hip", "decode_valu.hip", "dispatch.hip", "kernel_common.h",
                  "launch.h")


def kernel_source_sha() -> str:
    """Hash of the decode kernels' sources (kernels, shared header, launch)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def decode_kernel_name(w) -> str:
    mfma = w.head_dim == 128 and (
        (w.q_dtype == "bf16" and w.kv_dtype in ("bf16", "e4m3", "e2m1", "i4"))
        or (w.q_dtype == "f16" and w.kv_dtype == "f16"))
    return "decode_mfma_kernel" if mfma else "decode_kernel"


def compute_dtype(w) -> str:
    """Operand type of the decode kernel's products: the MFMA kernel multiplies
    16-bit operands (bf16; fp16 for fp16 KV; e4m3, e2m1 and int4 codes widen to
    bf16 exactly) into fp32 accumulators; the vector-ALU kernel works in fp32."""
    if decode_kernel_name(w) != "decode_mfma_kernel":
        return "f32"
    return "f16" if w.kv_dtype == "f16" else "bf16"


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, command: str) -> dict:
    """Per-launch HBM bytes of the decode kernel from two rocprofv3 --pmc runs of
    this bench (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).

    Each counter is scaled by what it reads for kernels of known size in the
    same run: the library's calibration read of the 1 GiB flush buffer
    (FETCH_SIZE; the flush itself, a torch reduction, where a run has no
    calibration read) and the 1 GiB zero fill of that buffer (WRITE_SIZE).
    The calibration read reads 2.000 (units of 512 B) per KiB in every run;
    the flush's ratio moved between 2.000 and 2.06 from run to run, so it is
    kept as a cross-check only.
    """
    import csv

    def rows(path, counter):
        out = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
        return out

    gib_kib = float(1 << 20)
    fr = rows(fetch_csv, "FETCH_SIZE")
    wr = rows(write_csv, "WRITE_SIZE")
    flush_reads = [v for n, g, v in fr if n.startswith("reduce_kernel")]
    fills = [v for n, g, v in wr if n.startswith("vectorized_elementwise") and v > 0.5 * gib_kib]
    flush_scale = gib_kib / (sum(flush_reads) / len(flush_reads))
    w_scale = gib_kib / (sum(fills) / len(fills))
    cal_reads = [v for n, g, v in fr if n.startswith("stream_read_kernel")]
    cal_scale = gib_kib / (sum(cal_reads) / len(cal_reads)) if cal_reads else None
    f_scale = cal_scale if cal_scale else flush_scale
    dec_f = [v for n, g, v in fr if n.startswith("decode_")]
    dec_w = [v for n, g, v in wr if n.startswith("decode_")]
    fetch_b = sum(dec_f) / len(dec_f) * 1024 * f_scale
    write_b = sum(dec_w) / len(dec_w) * 1024 * w_scale
    return {
        "workload": workload,
        "kernel": next(n for n, g, v in fr if n.startswith("decode_")),
        "dispatches": len(dec_f),
        "fetch_kib_raw_mean": sum(dec_f) / len(dec_f),
        "write_kib_raw_mean": sum(dec_w) / len(dec_w),
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "fetch_scale_of_calibration_read": cal_scale,
        "fetch_scale_of_flush_read": flush_scale,
        "scale_reference": ("calibration read of the 1 GiB flush buffer (stream_read_kernel)"
                            if cal_scale else "1 GiB cache-flush read (reduce_kernel)")
                           + " for FETCH_SIZE; 1 GiB zero fill (vectorized_elementwise_kernel) "
                           "for WRITE_SIZE, same runs",
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "kernel_source_sha256": kernel_source_sha(),
        "command": command,
    }


def load_traffic(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def _oracle_request(w, item):
    """The oracle on one request already copied to host memory (one sample task)."""
    import numpy as np

    from oracle import attention

    qh, kvh, n, last, ks, vs = item
    return attention.decode(qh, kvh, np.array([0, n], np.int32), np.arange(n, dtype=np.int32),
                            np.array([last], np.int32), num_kv_heads=w.num_kv_heads,
                            q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, sm_scale=w.scale(),
                            k_scale=ks, v_scale=vs,
                            qo_indptr=np.array([0, qh.shape[0]], np.int32))


def _pool_worker(conn):
    """A single-threaded oracle worker: receive its requests, wait for the start
    signal, compute them, report the time taken."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    w, items, passes = conn.recv()
    _oracle_request(w, items[0]) if items else None  # imports and first-touch outside timing
    conn.send("ready")
    conn.recv()
    t0 = time.perf_counter()
    for _ in range(passes):
        for it in items:
            _oracle_request(w, it)
    conn.send(time.perf_counter() - t0)
    conn.close()


def _oracle_pool(w, items, workers: int, passes: int = 1) -> float:
    """Wall seconds for `workers` processes to run the oracle `passes` times on
    `items`, which are assigned longest first to the least-loaded worker
    before timing."""
    import multiprocessing as mp

    ctx = mp.get_context("spawn")  # fresh interpreters: no device state is inherited
    shares = [[] for _ in range(workers)]
    load = [0] * workers
    for it in sorted(items, key=lambda it: -it[1].nbytes):
        k = load.index(min(load))
        shares[k].append(it)
        load[k] += it[1].nbytes
    procs, conns = [], []
    try:
        for k in range(workers):
            parent, child = ctx.Pipe()
            p = ctx.Process(target=_pool_worker, args=(child,), daemon=True)
            p.start()
            procs.append(p)
            conns.append(parent)
        for c, share in zip(conns, shares):
            c.send((w, share, passes))
        for c in conns:
            if c.recv() != "ready":
                raise RuntimeError("oracle worker failed to start")
        t0 = time.perf_counter()
        for c in conns:
            c.send("go")
        for c in conns:
            c.recv()
        return time.perf_counter() - t0
    finally:
        for p in procs:
            p.join(timeout=60)
            if p.is_alive():
                p.terminate()


def cpu_baseline(dcase, w, budget_s: float = 12.0, keep_bytes: int = 2 << 30):
    """The oracle, as it stands, on whole requests of the same batch.

    Single thread: requests in batch order until about `budget_s` seconds of
    CPU work have been spent; a batch that takes less is run again, whole,
    until the budget is reached (so the rate rests on seconds of work).
    Parallel: the same requests (up to `keep_bytes` of host KV) again, spread
    by KV bytes over worker processes, one per core of this process's
    affinity mask up to 16 (the CPU share of one GPU on the measurement
    hosts; the mask's size and the host's core count are reported beside
    it), each single-threaded, repeated so that the pool works for about a
    quarter of the budget. Copying KV to the host and handing it to
    the workers is outside both timings.
    """
    from threadpoolctl import threadpool_limits

    import numpy as np
    import torch

    lens = dcase["kv_lens"]
    done_bytes = 0
    done = []
    kept = []
    kept_bytes = 0
    kept_kv = 0
    t_total = 0.0
    idx = dcase["indices"]
    with threadpool_limits(limits=1):
        for r in range(len(lens)):
            pages = torch.as_tensor(np.asarray(idx[int(dcase["indptr"][r]):int(dcase["indptr"][r + 1])],
                                               dtype=np.int64), device=dcase["kv"].device)
            kv = dcase["kv"].index_select(0, pages)
            if w.kv_dtype == "bf16":
                kvh = kv.view(torch.int16).cpu().numpy().view(np.uint16)
            elif w.kv_dtype in ("e4m3", "e2m1", "i4"):
                kvh = kv.cpu().numpy().view(np.uint8)
            else:
                kvh = kv.cpu().numpy()
            qo = dcase["qo_indptr"]
            q = dcase["q"][r:r + 1] if qo is None else dcase["q"][int(qo[r]):int(qo[r + 1])]
            qh = (q.view(torch.int16).cpu().numpy().view(np.uint16) if w.q_dtype == "bf16"
                  else q.cpu().numpy())
            ks = vs = None
            if w.kv_dtype == "e4m3":
                ks = dcase["k_scale"].index_select(0, pages).cpu().numpy()
                vs = dcase["v_scale"].index_select(0, pages).cpu().numpy()
            elif w.kv_dtype in ("e2m1", "i4"):
                ks = dcase["k_scale"].cpu().numpy()
                vs = dcase["v_scale"].cpu().numpy()
            item = (qh, kvh, len(pages), int(dcase["last_page_len"][r]), ks, vs)
            t0 = time.perf_counter()
            _oracle_request(w, item)
            t_total += time.perf_counter() - t0
            done.append(r)
            req_bytes = int(lens[r]) * w.num_kv_heads * w.head_dim * 2 * ELEM_BITS[w.kv_dtype] // 8
            done_bytes += req_bytes
            if kept_bytes + kvh.nbytes <= keep_bytes:
                kept.append(item)
                kept_bytes += kvh.nbytes
                kept_kv += req_bytes
            if t_total >= budget_s:
                break
        # a whole batch in less than the budget: further passes over it
        passes = 1
        if len(done) == len(lens) and len(kept) == len(done):
            while t_total < budget_s and passes < 100000:
                t0 = time.perf_counter()
                for it in kept:
                    _oracle_request(w, it)
                t_total += time.perf_counter() - t0
                done_bytes += kept_kv
                passes += 1
    gbs = done_bytes / t_total / 1e9

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(16, affinity, len(kept)))
    # one pass over `kept` takes about t_kept on one thread; aim for a quarter
    # of the budget of wall time on `workers` processes
    t_kept = t_total * kept_kv / max(1, done_bytes)
    par_passes = max(1, min(100000, math.ceil(0.25 * budget_s * workers / max(t_kept, 1e-9))))
    t_par = _oracle_pool(w, kept, workers, par_passes)
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(done)} of {len(lens)} requests ({int(sum(lens[done]))} KV tokens, "
                   f"all {w.num_qo_heads} query heads)"
                   + (f", {passes} passes" if passes > 1 else "")
                   + f", float64 numpy oracle, 1 thread, {t_total:.1f} s"),
        "ms_per_full_step_extrapolated": round(t_total / max(1, done_bytes) * kv_bytes_total(dcase, w)
                                               * 1e3, 1),
        "parallel": {
            "value": round(kept_kv * par_passes / t_par / 1e9, 4),
            "unit": "GB/s",
            "cores": workers,
            "affinity_cores": affinity,
            "host_cores": os.cpu_count(),
            "sample": (f"the first {len(kept)} of those requests"
                       + (f", {par_passes} passes" if par_passes > 1 else "")
                       + f", over {workers} single-threaded worker processes, {t_par:.2f} s"),
        },
    }


def kv_bytes_total(dcase, w):
    return kv_bytes(w, dcase)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="ragged_loguniform_bf16")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--warm-ref", action="store_true",
                    help="also time K back-to-back steps without cache flushes (reported "
                         "as warm_*; off by default so that every decode launch of a run is "
                         "cold and a profiler's per-kernel average matches the events)")
    ap.add_argument("--flat", action="store_true",
                    help="for a shared-prefix workload, run plain decode over every request's "
                         "full page list instead of the cascade (for comparison)")
    ap.add_argument("--fixed-capacity", action="store_true",
                    help="plan with fixed capacities (the graph-capturable launch shape)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays "
                         "(implies --fixed-capacity)")
    ap.add_argument("--wgs-per-cu", type=int, default=0,
                    help="cap on decode workgroups per compute unit (0: library default)")
    ap.add_argument("--separate-merge", action="store_true",
                    help="launch and time the decode and merge stages apart instead of one "
                         "run() with the merge folded into the decode kernel")
    ap.add_argument("--layers", type=int, default=1,
                    help="run() calls per step, one per layer, each over its own copy of the "
                         "KV pool and all with the step's one plan (one graph holds them all "
                         "with --graph); times are reported per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--balance", type=int, default=0)
    ap.add_argument("--min-chunk-pages", type=int, default=0)
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_decode_<config>.json from two rocprofv3 "
                         "--pmc runs of this bench and exit")
    ap.add_argument("--counter-command", default="",
                    help="the rocprofv3 command lines recorded with --summarize-counters")
    args = ap.parse_args(argv)

    if args.summarize_counters:
        t = summarize_counters(*args.summarize_counters, args.config, args.counter_command)
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        path = os.path.join(ROOT, "profiles", f"traffic_decode_{args.config}.json")
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path here has no multi-GPU "
              "sharding (run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_decode_plan_amd as pk
    from workloads import CONFIGS, device_case

    if args.config not in CONFIGS:
        print(f"unknown config {args.config}; choose from {list(CONFIGS)}", file=sys.stderr)
        return 2
    w = CONFIGS[args.config]
    seed = args.seed if args.seed is not None else list(CONFIGS).index(args.config) + 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name} seed {seed}", file=sys.stderr, flush=True)
    dcase = device_case(w, seed, dev, poison=False)
    torch.cuda.synchronize()
    if args.flat and w.shared_prefix is not None:
        import dataclasses
        w = dataclasses.replace(w, shared_prefix=None)  # same tables, read in full
    nbytes = kv_bytes(w, dcase)

    ws = torch.empty(pk.DEFAULT_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    q_dt = dcase["q"].dtype
    kv_dt = w.kv_dtype if w.kv_dtype in ("e4m3", "e2m1", "i4") else dcase["kv"].dtype
    cascade = w.shared_prefix is not None
    if cascade:
        # Two levels (shared prefixes once for all their requests' queries,
        # then each request's own pages) and the merge of their results.
        wrapper = pk.CascadeBatchDecodeWrapper(ws, "NHD")
        sh, un = dcase["shared"], dcase["unique"]
        sh_idx = torch.as_tensor(sh["indices"], dtype=torch.int32).to(dev)
        un_idx = torch.as_tensor(un["indices"], dtype=torch.int32).to(dev)

        def do_plan():
            wrapper.plan(sh["indptr"], sh_idx, sh["last_page_len"], dcase["group_qo_indptr"],
                         un["indptr"], un_idx, un["last_page_len"], w.num_qo_heads,
                         w.num_kv_heads, w.head_dim, w.page_size, q_data_type=q_dt,
                         kv_data_type=kv_dt, out_data_type=q_dt, sm_scale=w.scale(),
                         balance=args.balance, min_chunk_pages=args.min_chunk_pages)
            torch.cuda.synchronize()
    else:
        wrapper = pk.BatchDecodeWithPagedKVCacheWrapper(ws, "NHD")
        indices_dev = torch.as_tensor(dcase["indices"], dtype=torch.int32).to(dev)
        capacity = None
        if args.fixed_capacity or args.graph:
            # Capacities from the bounds of the plan rule: items <= query blocks +
            # slots * balance / Hkv; merge tasks <= q rows; partial rows <= items
            # times tokens per item.
            qo = dcase["qo_indptr"]
            rows = w.batch if qo is None else int(qo[-1])
            max_q = 1 if qo is None else int(np.diff(qo).max())
            probe = pk.plan_partition(dcase["indptr"], dcase["last_page_len"], w.num_qo_heads,
                                      w.num_kv_heads, w.head_dim, w.page_size,
                                      kv_dtype=w.kv_dtype, q_dtype=w.q_dtype, slots=1,
                                      qo_indptr=qo)[0]
            items = rows + 4096 * max(1, args.balance) // w.num_kv_heads
            capacity = dict(items=items, merge_tasks=rows,
                            partials=items * probe["queries_per_item"], qo_len=max_q)

        def do_plan():
            wrapper.plan(dcase["indptr"], indices_dev, dcase["last_page_len"], w.num_qo_heads,
                         w.num_kv_heads, w.head_dim, w.page_size, q_data_type=q_dt,
                         kv_data_type=kv_dt, out_data_type=q_dt, sm_scale=w.scale(),
                         balance=args.balance, min_chunk_pages=args.min_chunk_pages,
                         qo_indptr=dcase["qo_indptr"], capacity=capacity,
                         max_wgs_per_cu=args.wgs_per_cu, kv_scale=w.kv_scale)
            torch.cuda.synchronize()

    t0 = time.perf_counter()
    do_plan()  # first plan of the process: device query and staging allocation
    first_plan_us = (time.perf_counter() - t0) * 1e6
    plan_times = []
    for _ in range(9):  # steady state: one plan per step, shared by every layer's run()
        t0 = time.perf_counter()
        do_plan()
        plan_times.append((time.perf_counter() - t0) * 1e6)
    plan_us = statistics.median(plan_times)
    if cascade:
        levels = [lv.plan_info for lv in wrapper._levels]
        info = dict(levels[1])
        info["levels"] = levels
    else:
        info = wrapper.plan_info
    out = torch.empty_like(dcase["q"])
    run_kw = dict(out=out, k_scale=dcase["k_scale"], v_scale=dcase["v_scale"])
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_i64 = flush.view(torch.int64)
    flush.zero_()

    from paged_kv_decode_plan_amd import _lib

    # By default a step is one run(): the decode kernel with the merge of split
    # requests folded in. --separate-merge times the two stages apart instead.
    has_merge = (args.separate_merge and not cascade and args.layers == 1
                 and info["num_split_requests"] > 0)
    if args.layers < 1 or (args.layers > 1 and cascade):
        print("--layers takes a count >= 1 and single-plan workloads only", file=sys.stderr)
        return 2
    # One KV pool per layer (the first is the generated one): every layer's
    # run() reads its own bytes, as in a model, so no layer finds the previous
    # one's KV in the caches.
    kv_layers = [dcase["kv"]] + [dcase["kv"].clone() for _ in range(args.layers - 1)]
    graph = None
    if args.graph:
        if cascade:
            print("--graph covers single-plan workloads only", file=sys.stderr)
            return 2
        wrapper.run(dcase["q"], dcase["kv"], **run_kw)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for kv in kv_layers:
                wrapper.run(dcase["q"], kv, **run_kw)
        torch.cuda.synchronize()
        has_merge = False

    def step(ev=None, kernel_ev=None):
        """One run(). Timed steps bracket it with events; with --separate-merge
        the decode and merge stages are launched and bracketed apart (an event
        pair costs a few µs itself)."""
        if graph is not None:  # decode and merge kernels replayed from the graph
            if ev is not None:
                ev[0].record()
            graph.replay()
            if ev is not None:
                ev[1].record()
            return
        if kernel_ev is not None:  # events stamped by the decode kernel's own dispatch
            if has_merge:
                wrapper.run(dcase["q"], dcase["kv"], stages=_lib.STAGE_DECODE,
                            decode_events=kernel_ev, **run_kw)
                wrapper.run(dcase["q"], dcase["kv"], stages=_lib.STAGE_MERGE, **run_kw)
            else:
                wrapper.run(dcase["q"], dcase["kv"], decode_events=kernel_ev, **run_kw)
            return
        if ev is None:
            for kv in kv_layers:
                wrapper.run(dcase["q"], kv, **run_kw)
            return
        if not has_merge:  # one bracket around the whole run (every layer's)
            ev[0].record()
            for kv in kv_layers:
                wrapper.run(dcase["q"], kv, **run_kw)
            ev[1].record()
            return
        ev[0].record()
        wrapper.run(dcase["q"], dcase["kv"], stages=_lib.STAGE_DECODE, **run_kw)
        ev[1].record()
        if has_merge:
            wrapper.run(dcase["q"], dcase["kv"], stages=_lib.STAGE_MERGE, **run_kw)
            ev[2].record()

    print(f"[bench] plan {info}; warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        if not args.warm:
            flush_i64.max()
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        if not args.warm:
            flush_i64.max()  # read 1 GiB: evict KV from L2 and the last-level cache
        step(evs[i])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    bracket_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = bracket_ms
    # Decode kernel time: a second series of as many cold steps whose decode
    # launches record events in the kernel's own dispatch (hipExtLaunchKernel).
    # Events around a launch add the queue's packet overhead (a few µs), and
    # the dispatch-stamped ones slow the launch itself, so each series times
    # one thing: the steps above, the kernel here. A cascade step (several
    # launches) and a graph replay keep the bracket.
    kernel_events = graph is None and not cascade and args.layers == 1
    if kernel_events:
        kevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in kevs:  # create the events before the timed series
            e[0].record()
            e[1].record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            if not args.warm:
                flush_i64.max()
            step(kernel_ev=kevs[i])
        torch.cuda.synchronize()
        dec_ms = [e[0].elapsed_time(e[1]) for e in kevs]
    mrg_ms = [e[1].elapsed_time(e[2]) for e in evs] if has_merge else [0.0]
    step_ms = [e[0].elapsed_time(e[2 if has_merge else 1]) for e in evs]
    if args.layers > 1:  # per layer
        step_ms = [t / args.layers for t in step_ms]
        bracket_ms = [t / args.layers for t in bracket_ms]
        dec_ms = bracket_ms
    print(f"[bench] timed {args.steps} steps in {wall_s:.2f} s", file=sys.stderr, flush=True)

    # Calibration: the library's plain streaming read over the 1 GiB flush
    # buffer, at 1, 2 and 4 workgroups per compute unit (median of 10 each).
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    cal = {}
    sink = torch.empty(4 * 4 * cus, dtype=torch.int32, device=dev)
    for per_cu in (1, 2, 4):
        pk.stream_read(flush, per_cu * cus, sink)  # warm the launch path
        cal_ms = []
        for _ in range(10):
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            pk.stream_read(flush, per_cu * cus, sink)
            c1.record()
            torch.cuda.synchronize()
            cal_ms.append(c0.elapsed_time(c1))
        cal[per_cu] = flush.numel() / (statistics.median(cal_ms) * 1e-3) / 1e9
    best_cal = max(cal, key=cal.get)
    cal_gbs = cal[best_cal]

    warm_ms = None
    if args.warm_ref:  # back-to-back steps, for reference
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        warm_ms = e0.elapsed_time(e1) / args.steps / args.layers

    mean_step = statistics.fmean(step_ms)
    mean_dec = statistics.fmean(dec_ms)
    q = statistics.quantiles(step_ms, n=10) if len(step_ms) >= 2 else [mean_step] * 9
    gbs = nbytes / (mean_step * 1e-3) / 1e9
    dec_gbs = nbytes / (mean_dec * 1e-3) / 1e9
    traffic = load_traffic(w.name)

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(w),
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "num_qo_heads": w.num_qo_heads,
            "query_tokens": int(info["query_rows"]),
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
            "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype, "context": list(w.context),
            "total_kv_tokens": int(dcase["kv_lens"].sum()), "seed": seed,
            "cache": "warm" if args.warm else "cold (1 GiB read between steps)",
            "layers": args.layers,
            "launch": ("hip graph replay, fixed-capacity plan" if args.graph else
                       "fixed-capacity plan" if args.fixed_capacity else "exact plan"),
        },
        "us_per_step": round(mean_step * 1e3, 2),
        "us_per_step_median": round(statistics.median(step_ms) * 1e3, 2),
        "us_per_step_p10_p90": [round(q[0] * 1e3, 2), round(q[-1] * 1e3, 2)],
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "kv_bytes_per_step": nbytes,
        "warm_us_per_step": round(warm_ms * 1e3, 2) if warm_ms else None,
        "warm_gbs": round(nbytes / (warm_ms * 1e-3) / 1e9, 1) if warm_ms else None,
        # timed apart only with --separate-merge; otherwise inside the step
        "merge_us": round(statistics.fmean(mrg_ms) * 1e3, 2) if has_merge else None,
        "merge": ("none (no request split)" if info["num_split_requests"] == 0 else
                  "separate stages (timed apart)" if has_merge else
                  "folded into the decode kernel" if info.get("merge_folded") else
                  "separate merge kernel inside the step"),
        "calibration": {
            "kernel": ("stream_read_kernel (pkd_stream_read): plain streaming read of a 1 GiB "
                       "buffer, 16-byte non-temporal loads, 8 KiB in flight per wavefront"),
            "read_gbs": round(cal_gbs, 1),
            "pct_of_peak_hbm": round(100.0 * cal_gbs / PEAK_HBM_GBS, 2),
            "workgroups_per_cu": best_cal,
            "read_gbs_by_workgroups_per_cu": {str(k): round(v, 1) for k, v in cal.items()},
            "decode_kernel_over_calibration": round(dec_gbs / cal_gbs, 4),
        },
        "plan_us_host": round(plan_us, 1),
        "plan_us_host_first": round(first_plan_us, 1),
        "plan": ({"levels": [{k: lv[k] for k in PLAN_KEYS} for lv in info["levels"]]}
                 if cascade else {k: info[k] for k in PLAN_KEYS}),
        "roofline": {
            "kernel": ("cascade step: prefix-level and suffix-level " + decode_kernel_name(w)
                       + " with their merges and merge_states" if cascade
                       else decode_kernel_name(w)),
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "decode_us": round(mean_dec * 1e3, 2),
            "decode_timing": ("events recorded by the decode kernel's dispatch (hipExtLaunchKernel), "
                              f"{args.steps} more cold steps" if kernel_events
                              else "events around the step" if args.layers == 1
                              else f"events around the step's {args.layers} layers, divided by "
                                   f"{args.layers}"),
            "decode_bracket_us": round(statistics.fmean(bracket_ms) * 1e3, 2),
            "algorithmic_bytes_per_launch": nbytes,
        },
    }
    if cascade:
        logical = kv_bytes(w, dcase, logical=True)
        result["cascade"] = {
            "shared_prefix": list(w.shared_prefix),
            "logical_kv_bytes_per_step": logical,
            "logical_kv_gbs": round(logical / (mean_step * 1e-3) / 1e9, 1),
        }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(dcase, w, args.cpu_budget)
    wrapper.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
