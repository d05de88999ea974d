"""bench.py's command line without a GPU: more than one GPU is refused with a
message and exit status 2 before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], env=e,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    r = run_bench([], env={"WORLD_SIZE": "8"})
    assert r.returncode == 2 and "one GPU only" in r.stderr
