"""bench.py's command line on the host: its options parse, and a request for
more than one GPU is refused with a message before any device is touched (the
library has no multi-GPU path)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_help_lists_the_workload_options():
    r = _run("--help")
    assert r.returncode == 0, r.stderr
    for opt in ("--steps", "--warmup", "--config", "--repack-config", "--ns-tiles", "--ns-streams", "--gpus"):
        assert opt in r.stdout, opt


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
