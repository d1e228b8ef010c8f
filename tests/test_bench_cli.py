"""bench.py command-line contract checks that need no GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _run("--gpus", str(n))
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == n and "one GPU" in line["error"]


def test_help_lists_the_measurement_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--config", "--epilogue", "--seeding", "--zipf-update", "--tune", "--probe"):
        assert opt in r.stdout, opt
