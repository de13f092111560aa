"""GPU: seeded random shapes against the oracle, and guard zones around every output.

Each fuzz case draws dtype, head size, block size, query group, kernel family, partition size,
the fused newest-token write and a ragged batch whose lengths sit on block, chunk and partition
edges (and include empty contexts). The guard-zone tests surround `out` and each part of the
split-context workspace with canary bit patterns and check that no launch writes outside them.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL, bits, oracle_out, oracle_pools, out_f64, run_step, to_dev, to_host,
                      upload)
from paged_kv_cache_247_amd import workload as W
import paged_kv_cache_247_amd as pk

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    print(f"\n[gpu] {request.node.name}", file=sys.stderr, flush=True)


def fuzz_case(case: int):
    rng = np.random.default_rng(9000 + case)
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    D = int(rng.choice([64, 128]))
    S = int(rng.choice([16, 32, 64, 128, 256]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 8]))
    kernels = ["auto", "valu"] + (["mfma"] if dtype != "f32" else [])
    kernel = str(rng.choice(kernels))
    P = int(rng.choice([0, S, 2 * S, 512 if 512 % S == 0 else 2 * S]))
    B = int(rng.integers(1, 7))
    edges = [1, 2, S - 1, S, S + 1, 31, 32, 33, 2 * S + 3] + ([P - 1, P, P + 1] if P else [])
    lens = []
    for _ in range(B):
        u = rng.random()
        lens.append(0 if u < 0.1 else int(rng.choice(edges)) if u < 0.6
                    else int(rng.integers(1, 600)))
    if not any(lens):
        lens[0] = S + 1
    lens = np.array(lens, dtype=np.int32)
    fused = bool(rng.random() < 0.5)
    blocks = int(sum(-(-int(x) // S) for x in lens))
    cfg = W.SMALL["c3"].replace(name=f"fuzz{case}", num_seqs=B, num_heads=G * Hkv,
                                num_kv_heads=Hkv, head_dim=D, block_size=S, dtype=dtype,
                                num_blocks=blocks + 4, len_lo=1, len_hi=int(lens.max()),
                                seed=9000 + case, partition_size=P)
    return cfg, lens, kernel, P, fused


@pytest.mark.parametrize("case", range(30))
def test_random_shapes_match_oracle(case):
    cfg, lens, kernel, P, fused = fuzz_case(case)
    print(f"[gpu] fuzz {case}: {cfg.dtype} D{cfg.head_dim} S{cfg.block_size} "
          f"{cfg.num_heads}/{cfg.num_kv_heads} {kernel} P{P} fused={fused} lens={lens.tolist()}",
          file=sys.stderr, flush=True)
    wl = W.generate(cfg, lens=lens)
    kc, vc = oracle_pools(wl)
    ref = oracle_out(wl, pools=(kc, vc))
    dev = upload(wl)
    out = run_step(dev, wl, kernel=kernel, partition_size=P, fused=fused,
                   order=wl.work_items(P) if case % 2 else None)
    o = out_f64(out)
    assert not o[lens == 0].any(), "empty contexts give zeros"
    err = oracle.max_abs_err(o, ref)
    assert err <= TOL[cfg.dtype], f"max abs err {err}"
    assert np.array_equal(bits(to_host(dev.k, cfg.dtype)), bits(kc))
    assert np.array_equal(bits(to_host(dev.v, cfg.dtype)), bits(vc))


GUARD = 256  # elements of canary on each side


def guarded(shape, dtype, pattern: int):
    """A tensor of `shape` inside one allocation with GUARD canary elements on each side."""
    n = int(np.prod(shape))
    itype = {2: torch.int16, 4: torch.int32}[torch.empty(0, dtype=dtype).element_size()]
    buf = torch.empty(2 * GUARD + n, dtype=dtype, device="cuda")
    buf.view(itype).fill_(pattern)
    return buf, buf[GUARD:GUARD + n].view(shape), itype


def guards_intact(buf, itype, pattern: int):
    raw = buf.view(itype)
    return bool((raw[:GUARD] == pattern).all() and (raw[-GUARD:] == pattern).all())


@pytest.mark.parametrize("name,P,fused", [("c3", 0, True), ("c3", 0, False), ("c5", 64, True),
                                          ("c2", 32, False), ("c1", 16, True)])
def test_no_write_outside_out_or_workspace(name, P, fused):
    wl = W.generate(W.SMALL[name])
    c = wl.cfg
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c.dtype]
    d = upload(wl)
    if len(wl.block_mapping):
        pk.copy_blocks([d.k], [d.v], d.mapping)
    if not fused:
        pk.reshape_and_cache(d.key, d.value, d.k, d.v, d.slots)
    ob, out, oit = guarded((c.num_seqs, c.num_heads, c.head_dim), tdt, 0x5A5A)
    ws, wbufs = None, []
    if P:
        NP = pk.num_partitions(wl.max_context_len, P)
        parts = []
        for shp in ((c.num_seqs, c.num_heads, NP), (c.num_seqs, c.num_heads, NP),
                    (c.num_seqs, c.num_heads, NP, c.head_dim)):
            b, t, it = guarded(shp, torch.float32, 0x7FC0A5A5)
            wbufs.append((b, it))
            parts.append(t)
        ws = tuple(parts)
    pk.paged_attention(out, d.q, d.k, d.v, d.bt, d.lens, wl.max_context_len, c.scale, P, ws,
                       work_items=to_dev(wl.work_items(P)),
                       new_key=d.key if fused else None, new_value=d.value if fused else None)
    torch.cuda.synchronize()
    assert guards_intact(ob, oit, 0x5A5A), "a write landed outside out"
    for b, it in wbufs:
        assert guards_intact(b, it, 0x7FC0A5A5), "a write landed outside the workspace"
    kc, vc = oracle_pools(wl)
    assert oracle.max_abs_err(out_f64(out), oracle_out(wl, pools=(kc, vc))) <= TOL[c.dtype]


def test_sync_mode_runs_a_step(monkeypatch):
    """PKV_SYNC=1: every call waits for its work (a debugging aid); the step is unchanged."""
    wl = W.generate(W.SMALL["c5"])
    a = run_step(upload(wl), wl, fused=True)
    monkeypatch.setenv("PKV_SYNC", "1")
    b = run_step(upload(wl), wl, fused=True)
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
