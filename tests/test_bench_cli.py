"""bench.py's command line without a GPU: more than one GPU is refused with a
message, and a multi-rank launch likewise."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_multi_rank_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run([], env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr

