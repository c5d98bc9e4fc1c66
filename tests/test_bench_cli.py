"""bench.py command-line contract checks that need no GPU."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    # one context-parallel rank on one GPU: N > 1 is refused before any GPU work
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_exits_too():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2


def test_help_lists_the_contract_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--settle-ms", "--cpu-seconds"):
        assert flag in r.stdout
