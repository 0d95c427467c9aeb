"""bench.py's command-line contract, checked on the CPU (no kernel runs)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_a_multi_rank_launch_is_refused_with_a_message():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _bench(env=env)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""
