"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner and the C ABI (``planner.cpp``, ``capi.cpp``) and a test program
(``tests/sanitize/host_paths.cpp``) are compiled for the host only with both
sanitizers; the kernel translation units are linked from the regular build's
objects (their device code is not run: no kernel is launched). The test
program then

* builds partitions of seeded tables through the C++ planner directly, which
  this test compares bit for bit with the float64 oracle's rule, including
  several resident workgroups per compute unit (``slots_per_cu`` 1-4, which
  the C ABI sets only from a device query), several query tokens per request
  and the non-causal shared-prefix level;
* drives the C ABI's host paths: plans of random tables, their info and work
  lists, every argument check that fails before a HIP call, and plans made
  from eight threads at once.

Any sanitizer report (out-of-bounds access, use after free, leak, undefined
behaviour) fails the test. CPU only.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import plan as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_decode_plan_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
# every device-code translation unit of the library (all of csrc/*.hip)
KERNEL_TUS = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
ENV = {
    "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=86",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
}


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _kernel_object(name, tmp):
    """The regular build's object of a kernel translation unit when it is newer
    than every device source, else a fresh compile of it into `tmp`."""
    obj = os.path.join(BUILD, name + ".o")
    newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
    if os.path.exists(obj) and os.path.getmtime(obj) >= newest:
        return obj
    from paged_kv_decode_plan_amd import build as pb
    out = os.path.join(tmp, name + ".o")
    cmd = [_hipcc(), *pb.COMMON, "-c", os.path.join(CSRC, name), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


@pytest.fixture(scope="module")
def sanitized_program(tmp_path_factory):
    if not os.path.exists(_hipcc()):
        pytest.skip("hipcc is not installed")
    tmp = str(tmp_path_factory.mktemp("sanitize"))
    host = {"planner.cpp": os.path.join(CSRC, "planner.cpp"),
            "capi.cpp": os.path.join(CSRC, "capi.cpp"),
            "host_paths.cpp": os.path.join(ROOT, "tests", "sanitize", "host_paths.cpp")}
    objs = []
    for name, src in host.items():
        obj = os.path.join(tmp, name + ".o")
        cmd = [_hipcc(), "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
               *SANITIZE, "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
               "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        objs.append(obj)
    objs += [_kernel_object(n, tmp) for n in KERNEL_TUS]
    exe = os.path.join(tmp, "host_paths")
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin",
                         "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    res = subprocess.run([clang, "-fsanitize=address,undefined", *objs, "-o", exe,
                          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def _run(exe, mode, stdin=""):
    env = dict(os.environ, **ENV)
    res = subprocess.run([exe, mode], input=stdin, capture_output=True, text=True, env=env,
                         timeout=300)
    assert "Sanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr
    assert res.returncode == 0, (res.returncode, res.stderr[-4000:])
    return res.stdout


def _cases():
    """Seeded partition inputs: free random tables, near-equal batches, single
    requests, several query tokens per request and non-causal rows, with 1-4
    slots per compute unit."""
    rng = np.random.default_rng(31337)
    cases = []
    for i in range(240):
        kind = i % 6
        P = int(rng.choice([1, 4, 16, 64]))
        if kind in (0, 3, 4, 5):
            B = int(rng.integers(1, 120))
            n = rng.integers(1, int(rng.integers(2, 400)), size=B)
        elif kind == 1:
            B = int(rng.integers(2, 300))
            N = int(rng.integers(1, 400))
            n = rng.integers(N - N // 9, N + 1, size=B)
            n[0] = N
        else:
            B, n = 1, np.array([int(rng.integers(1, 6000))])
        indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
        last = rng.integers(1, P + 1, size=B)
        L = (n - 1) * P + last
        qo, qpi, causal = None, 1, True
        if kind in (3, 4):
            nq = np.minimum(rng.integers(1, 40, size=B), L)
            qo = np.concatenate([[0], np.cumsum(nq)])
            qpi = int(rng.integers(1, 17))
        if kind == 5:
            nq = rng.integers(1, 60, size=B)
            qo = np.concatenate([[0], np.cumsum(nq)])
            qpi, causal = int(rng.integers(1, 17)), False
        cases.append(dict(indptr=indptr, last=last, P=P, units=int(rng.choice([1, 2, 4, 8])),
                          slots=int(rng.integers(1, 4096)), per_cu=int(rng.integers(1, 5)),
                          balance=int(rng.integers(1, 5)), cmin=int(rng.integers(1, 40)),
                          causal=causal, qpi=qpi, qo=qo))
    return cases


def _encode(cases):
    lines = [str(len(cases))]
    for c in cases:
        B = len(c["last"])
        lines.append(" ".join(map(str, [B, c["P"], c["units"], c["slots"], c["per_cu"],
                                        c["balance"], c["cmin"], int(c["causal"]), c["qpi"],
                                        int(c["qo"] is not None)])))
        lines.append(" ".join(map(str, c["indptr"])))
        lines.append(" ".join(map(str, c["last"])))
        if c["qo"] is not None:
            lines.append(" ".join(map(str, c["qo"])))
    return "\n".join(lines) + "\n"


def test_planner_under_sanitizers_matches_the_oracle(sanitized_program):
    cases = _cases()
    out = _run(sanitized_program, "partition", _encode(cases)).splitlines()
    pos = 0
    per_cu_seen = set()
    for c in cases:
        head = out[pos].split()
        pos += 1
        assert head[0] == "ok", out[pos - 1]
        C, n_items, n_partials, n_split = map(int, head[1:])
        items = np.array([list(map(int, out[pos + i].split())) for i in range(n_items)],
                         dtype=np.int32).reshape(-1, 8)
        pos += n_items
        merge = np.array(out[pos].split(), dtype=np.int32)
        split = np.array(out[pos + 1].split(), dtype=np.int32)
        pos += 2
        ref = oplan.plan(c["indptr"], c["last"], c["P"], c["units"], c["slots"], c["balance"],
                         c["cmin"], c["qo"], c["qpi"], causal=c["causal"],
                         slots_per_cu=c["per_cu"])
        assert C == ref["chunk_pages"]
        assert np.array_equal(items, ref["items"])
        assert np.array_equal(merge, ref["merge_indptr"])
        assert np.array_equal(split, ref["split_requests"])
        assert n_partials == ref["num_partials"]
        per_cu_seen.add(c["per_cu"])
    assert pos == len(out)
    assert per_cu_seen == {1, 2, 3, 4}


def test_planner_rejects_bad_tables_under_sanitizers(sanitized_program):
    bad = [dict(indptr=[0, 0], last=[1]), dict(indptr=[0, 2], last=[0]),
           dict(indptr=[0, 2], last=[17]), dict(indptr=[1, 2], last=[1])]
    cases = [dict(indptr=np.array(b["indptr"]), last=np.array(b["last"]), P=16, units=1,
                  slots=8, per_cu=1, balance=1, cmin=1, causal=True, qpi=1, qo=None)
             for b in bad]
    out = _run(sanitized_program, "partition", _encode(cases)).splitlines()
    assert len(out) == len(bad) and all(line.startswith("err ") for line in out)


def test_c_abi_host_paths_under_sanitizers(sanitized_program):
    assert "abi checks: 0 failures" in _run(sanitized_program, "abi")
