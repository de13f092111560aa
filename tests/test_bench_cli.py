"""bench.py's refusals, which happen before any data is generated or any GPU is touched: more
than one GPU, shard specifications that do not divide the workload, unsupported block
sizes; and the gating of the recorded HBM traffic on the launch it was measured on."""
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



def _summary(name):
    vals = {}
    for line in open(os.path.join(ROOT, "profiles", f"decode_{name}_counters.txt")):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def _sha(sources):
    import hashlib
    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_247_amd", "csrc", src), "rb").read())
    return h.hexdigest()


@pytest.mark.parametrize("name,family,mode", [("c2", "valu", False), ("c3", "mfma", False),
                                              ("c4", "mfma", "whole"), ("c5", "mfma", False)])
def test_counter_traffic_is_gated_on_sources_mode_and_partition_size(name, family, mode):
    """The HBM traffic of a profiled launch is reported only for the kernel sources, decode mode
    (grouped shared-prefix launches or not) and partition size it was taken with. Each committed
    summary records the benchmark's own launch of its workload; whether its sources are still
    current decides only whether that launch reads the recorded figure."""
    sys.path.insert(0, ROOT)
    import bench
    vals = _summary(name)
    _, P, _ = bench.LAUNCH[name]
    assert vals.get("partition_size", "0") == str(P)
    assert vals.get("shared_prefix", "0") == (mode if isinstance(mode, str) else "0")
    src = bench.KERNEL_SOURCES[family]
    got = bench.counter_traffic(src, name, mode, P)
    if vals["source_sha256"] == _sha(src):
        assert got == int(float(vals["traffic_bytes_per_launch"]))
    else:
        assert got is None
    assert bench.counter_traffic(src, name, mode, P + 16) is None
    assert bench.counter_traffic(src, name, "whole" if mode is False else False, P) is None
    other = bench.KERNEL_SOURCES["mfma" if family == "valu" else "valu"]
    assert bench.counter_traffic(other, name, mode, P) is None


def test_unknown_between_launches_work_is_refused():
    r = run("--config", "c3", "--between-launches", "everything", "--no-cpu-baseline")
    assert r.returncode == 2 and "--between-launches" in r.stderr and not r.stdout
