"""bench.py's command line on the host: it measures one GPU and says so when
asked for more, before touching torch or a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*argv, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          capture_output=True, text=True, timeout=60, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused_too():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _bench("--gpus", "1", env=env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
