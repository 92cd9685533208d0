"""bench.py's command-line contract, checked without a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_exits_with_a_message():
    """The step is one rank's shard on one GPU: --gpus N > 1 prints one
    JSON line saying so and exits non-zero, before touching a GPU."""
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
    assert "one GPU" in r.stderr


def test_help_lists_the_driver_flags():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout
