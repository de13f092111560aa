"""bench.py's refusals, which happen before any data is generated or any GPU is touched: more
than one GPU, shard specifications that do not divide the workload, unsupported block
sizes."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr and not r.stdout


@pytest.mark.parametrize("spec", ["kv:3", "seq:7", "heads:2", "kv:0", "kv:16"])
def test_bad_shards_are_refused(spec):
    r = run("--config", "c3", "--shard", spec, "--no-cpu-baseline")
    assert r.returncode == 2 and "--shard" in r.stderr and not r.stdout


@pytest.mark.parametrize("S", ["8", "48", "512"])
def test_unsupported_block_sizes_are_refused(S):
    r = run("--config", "c3", "--block-size", S, "--no-cpu-baseline")
    assert r.returncode == 2 and "--block-size" in r.stderr and not r.stdout
