"""Paged decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3] [--kernel auto]
                    [--partition-size P] [--unfused] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch: copy-on-write block copies (when
the workload has them), the cache write of each sequence's newest token, paged decode, and the
partition merge when the context is split. By default the cache write is fused into the decode
launch (--unfused writes with a separate reshape_and_cache launch). Inputs are resident in HBM
before timing starts.

Prints one JSON line: KV-read GB/s over the step (value), attended tokens/s, the decode
kernel's roofline figures (timed per launch with HIP events on the launch stream), repetition
statistics of back-to-back launches of each kernel on its own (decode, cache write, block copy,
merge), and the oracle's CPU throughput on the same workload at one thread and at all cores.
The oracle is timed first, before anything touches the GPU, so its worker processes are plain
CPU processes.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix-core peak, AMD published

# Launch configuration the benchmark uses for each workload: (kernel family, partition size,
# cached K/V loads). With longest-first dispatch, single-pass decode is fastest up to 4k-token
# contexts; the lognormal long-context batch (up to ~31k tokens) splits into 2048-token
# partitions; the prefix-shared batch keeps K/V in cache so the shared prefix is reused.
LAUNCH = {
    "c1": ("auto", 0, False),
    "c2": ("auto", 0, False),
    "c3": ("auto", 0, False),
    "c4": ("auto", 0, True),
    "c5": ("auto", 2048, False),
}

BLOCK_SIZES = (16, 32, 64, 128, 256)  # block sizes the library takes

# Sources the decode kernels are built from (a change to any invalidates counter figures).
KERNEL_SOURCES = {"mfma": ["decode_mfma.hip", "common.hpp", "kernels.hpp"],
                  "valu": ["decode_valu.hip", "common.hpp", "kernels.hpp"]}


def parse():
    ap = argparse.ArgumentParser(description="paged decode benchmark (one GPU)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", choices=sorted(LAUNCH) + ["p1", "p2"],
                    help="c1..c5: decode workloads; p1, p2: prefill workloads")
    ap.add_argument("--kernel", default=None, choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--unfused", action="store_true",
                    help="write new tokens with a separate reshape_and_cache launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time to spend timing the oracle on one thread")
    ap.add_argument("--cpu-all-seconds", type=float, default=3.0,
                    help="wall time to spend timing the oracle on all cores")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: the host's cores, at most 16)")
    ap.add_argument("--reps", type=int, default=5,
                    help="repetitions of back-to-back launch timing per kernel")
    ap.add_argument("--launches", type=int, default=100,
                    help="back-to-back launches per repetition")
    ap.add_argument("--shared-prefix", default="auto", choices=["auto", "on", "off"],
                    help="decode blocks that sequences share once per group of sequences "
                         "(auto: when the batch shares a prefix and runs single pass)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="run the workload in blocks of this many positions (16..256); the "
                         "pool keeps at least its capacity")
    ap.add_argument("--shard", default=None, metavar="KIND:N",
                    help="run one GPU's share of an N-GPU job at its real shape: kv:N keeps "
                         "1/N of the kv heads (and their q heads), seq:N 1/N of the sequences")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ oracle on the CPU

_WL = None  # the workload, inherited by forked oracle workers


def _oracle_part(idx):
    """One worker's share of an oracle pass: decode of the sequences idx on one thread."""
    from threadpoolctl import threadpool_limits

    import oracle
    c = _WL.cfg
    with threadpool_limits(limits=1):
        oracle.decode(_WL.q[idx], _WL.k_cache, _WL.v_cache, _WL.block_tables[idx],
                      _WL.context_lens[idx], c.scale, c.num_kv_heads, c.dtype)
    return int(_WL.context_lens[idx].sum())


def _shares(lens, n):
    """Sequence index sets for n workers, longest first onto the least loaded."""
    load = [0] * n
    parts = [[] for _ in range(n)]
    for i in np.argsort(-lens, kind="stable"):
        k = int(np.argmin(load))
        parts[k].append(int(i))
        load[k] += int(lens[i])
    return [np.array(sorted(p), dtype=np.int64) for p in parts if p]


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, one_s: float, all_s: float, workers: int):
    """The oracle's decode (fp64 numpy) over whole passes of the workload: first on one thread
    for about one_s seconds, then split over `workers` forked processes (one thread each) for
    about all_s seconds of wall time."""
    global _WL
    from threadpoolctl import threadpool_limits

    import oracle
    c = wl.cfg
    elt = 4 if c.dtype == "f32" else 2
    per_tok = c.num_kv_heads * c.head_dim * elt * 2
    passes, toks, dt = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while dt < one_s:
            t0 = time.perf_counter()
            oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                          c.scale, c.num_kv_heads, c.dtype)
            dt += time.perf_counter() - t0
            passes += 1
            toks += wl.total_tokens
    res = {"value": round(toks * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"{passes} whole passes over all {c.num_seqs} sequences ({wl.total_tokens} "
                     f"context tokens each), fp64 numpy decode on one thread, {dt:.1f} s",
           "attended_tokens_per_s": round(toks / dt, 1),
           "cpu": cpu_model(), "host_cpus": os.cpu_count()}
    if workers > 1 and all_s > 0:
        _WL = wl
        shares = _shares(wl.context_lens, workers)
        with mp.get_context("fork").Pool(len(shares)) as pool:
            pool.map(_oracle_part, shares)  # start-up and first touch, untimed
            passes, toks = 0, 0
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < all_s:
                toks += sum(pool.map(_oracle_part, shares))
                passes += 1
            dt = time.perf_counter() - t0
        _WL = None
        res["all_cores"] = {
            "value": round(toks * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": len(shares),
            "sample": f"{passes} whole passes split over {len(shares)} processes (one thread "
                      f"each, sequences balanced by length), {dt:.1f} s wall",
            "attended_tokens_per_s": round(toks / dt, 1)}
    return res


# ------------------------------------------------------------------ GPU helpers

def counter_traffic(kernel_sources, workload, shared=False):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if the summary
    was taken on the kernel sources as they are now and in the same decode mode (the grouped
    shared-prefix launches or not), else None."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"decode_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in kernel_sources:
        h.update(open(os.path.join(root, "paged_kv_cache_247_amd", "csrc", src), "rb").read())
    if vals.get("source_sha256") != h.hexdigest():
        return None
    if int(vals.get("shared_prefix", "0")) != int(bool(shared)):
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def launch_stats(torch, fn, launches: int, reps: int, warmup: int = 10):
    """Microseconds per launch of fn over `reps` repetitions of `launches` back-to-back
    launches, bracketed by HIP events on the current stream: median, min, max."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / launches)
    per.sort()
    return {"median_us": round(per[len(per) // 2], 3), "min_us": round(per[0], 3),
            "max_us": round(per[-1], 3), "launches": launches, "reps": reps}


def prefill_cpu_baseline(wl, one_s: float):
    """The prefill oracle (fp64 numpy, one thread) over whole sequences of the workload,
    longest contexts first, until about one_s seconds have run."""
    from threadpoolctl import threadpool_limits

    import oracle
    c = wl.cfg
    done, flops, dt = 0, 0, 0.0
    with threadpool_limits(limits=1):
        for i in np.argsort(-wl.context_lens, kind="stable"):
            if dt >= one_s:
                break
            L, Q = int(wl.context_lens[i]), int(wl.query_lens[i])
            r0 = int(wl.query_start[i])
            t0 = time.perf_counter()
            oracle.prefill(wl.q_prefill[r0:r0 + Q], wl.k_cache, wl.v_cache,
                           wl.block_tables[i:i + 1], wl.context_lens[i:i + 1],
                           np.array([0, Q], dtype=np.int32), c.scale, c.num_kv_heads, c.dtype)
            dt += time.perf_counter() - t0
            done += 1
            flops += (2 * (L - Q) + Q + 1) * Q // 2 * c.num_heads * c.head_dim * 4
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {c.num_seqs} sequences (longest contexts first), fp64 numpy "
                      f"prefill on one thread, {dt:.1f} s",
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}


def prefill_main(args):
    """Prefill workloads: one step is the prefill attention launch over every sequence's new
    tokens (their K/V already in the cache), work units largest first."""
    import torch

    import paged_kv_cache_247_amd as pk
    from paged_kv_cache_247_amd import workload as W

    cfg = W.PREFILL[args.config]
    if args.block_size and args.block_size != cfg.block_size:
        cfg = cfg.with_block_size(args.block_size)
    wl = W.generate(cfg, poison="zero")
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(wl, args.cpu_seconds)
    pk.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, kc, vc = dev(wl.q_prefill), dev(wl.k_cache), dev(wl.v_cache)
    bt, lens, qs = dev(wl.block_tables), dev(wl.context_lens), dev(wl.query_start)
    out = torch.empty_like(q)
    tile = pk.prefill_tile_tokens(cfg.num_heads, cfg.num_kv_heads)
    order = dev(wl.prefill_work_items(tile))
    maxq = int(wl.query_lens.max())

    def prefill():
        pk.paged_attention_prefill(out, q, kc, vc, bt, lens, qs, maxq, cfg.scale,
                                   work_items=order)

    kernels = {"paged_attention_prefill": launch_stats(torch, prefill, args.launches, args.reps)}
    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    # The step is the prefill launch alone: one event pair brackets the timed region.
    t0 = time.perf_counter()
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    span[0].record()
    for _ in range(args.steps):
        prefill()
    span[1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    launch_ms = span[0].elapsed_time(span[1]) / args.steps
    fl = wl.prefill_flops()
    kernels["paged_attention_prefill"]["TFLOP_per_s"] = round(
        fl / (kernels["paged_attention_prefill"]["median_us"] * 1e-6) / 1e12, 2)
    line = {
        "metric": "paged prefill TFLOP/s (% of MI355X bf16 matrix-core peak) + query tokens/s",
        "value": round(fl / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "num_seqs": cfg.num_seqs,
                   "num_heads": cfg.num_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "block_size": cfg.block_size, "seed": cfg.seed,
                   "query_tokens": int(wl.query_start[-1]), "context_tokens": wl.total_tokens,
                   "flops": fl, "tile_tokens": tile, "work_units": int(len(order))},
        "query_tokens_per_s": round(int(wl.query_start[-1]) / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(fl / (launch_ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fl / (launch_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_attention_prefill",
                     "ms_per_launch": round(launch_ms, 5), "flops_per_launch": fl},
        "kernels": kernels,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the "
              "path runs on one GPU; --shard runs one GPU's share of a larger job)", file=sys.stderr)
        sys.exit(2)
    if args.block_size is not None and args.block_size not in BLOCK_SIZES:
        print(f"--block-size {args.block_size}: supported block sizes are {BLOCK_SIZES}",
              file=sys.stderr)
        sys.exit(2)
    if args.config in ("p1", "p2"):
        prefill_main(args)
        return
    from paged_kv_cache_247_amd import workload as W

    name = args.config
    kernel, P, cached = LAUNCH[name]
    kernel = args.kernel or kernel
    P = P if args.partition_size is None else args.partition_size
    cfg = W.CONFIGS[name]
    if args.block_size and args.block_size != cfg.block_size:
        cfg = cfg.with_block_size(args.block_size)
    shard = None
    if args.shard:
        kind, _, n = args.shard.partition(":")
        n = int(n)
        if kind == "kv" and n >= 1 and cfg.num_kv_heads % n == 0:
            cfg = cfg.replace(num_heads=cfg.num_heads // n, num_kv_heads=cfg.num_kv_heads // n)
        elif kind == "seq" and n >= 1 and cfg.num_seqs % n == 0:
            cfg = cfg.replace(num_seqs=cfg.num_seqs // n)
        else:
            print(f"--shard {args.shard}: expected kv:N (N dividing {cfg.num_kv_heads}) or "
                  f"seq:N (N dividing {cfg.num_seqs})", file=sys.stderr)
            sys.exit(2)
        shard = {"kind": kind, "of_gpus": n}
        cfg = cfg.replace(description=f"{cfg.description}; one GPU's share of {args.shard} "
                                      f"({cfg.num_seqs} seqs, {cfg.num_heads}/"
                                      f"{cfg.num_kv_heads} heads)")
    t0 = time.time()
    wl = W.generate(cfg, poison="zero")
    print(f"[bench] generated {name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        print(f"[bench] timing the oracle on the CPU (1 thread, then {workers} processes)",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds, args.cpu_all_seconds, workers)

    import torch

    import paged_kv_cache_247_amd as pk
    pk.load()  # fails loudly when the library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def dev(a, bf=False):
        a = np.ascontiguousarray(a)
        if bf:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    bf = cfg.dtype == "bf16"
    q, kc, vc = dev(wl.q, bf), dev(wl.k_cache, bf), dev(wl.v_cache, bf)
    key, value = dev(wl.key, bf), dev(wl.value, bf)
    slots, bt, lens = dev(wl.slot_mapping), dev(wl.block_tables), dev(wl.context_lens)
    mapping = dev(wl.block_mapping.reshape(-1, 2))
    fused = not args.unfused
    # Blocks shared by several sequences (a common prefix): plan groups that read each shared
    # tile once for all their members (host scheduler input, like the work list).
    plan = None
    if args.shared_prefix == "on" or (args.shared_prefix == "auto" and cfg.prefix_len and not P):
        from paged_kv_cache_247_amd import sharing
        plan = sharing.plan(wl.block_tables, wl.context_lens, cfg.block_size,
                            wl.max_context_len, cfg.group, newest_outside=fused)
        if plan is None and args.shared_prefix == "on":
            print("--shared-prefix on: no blocks are shared", file=sys.stderr)
            sys.exit(2)
    if plan is not None:
        P, kernel, cached = plan.partition_size, "mfma", True
        groups = dev(plan.groups)
        order = dev(plan.work_items)
    else:
        # Host-side scheduler input: the units with work, largest first.
        order = dev(wl.work_items(P))
    out = torch.empty((cfg.num_seqs, cfg.num_heads, cfg.head_dim), dtype=dt, device="cuda")
    ws = pk.partition_workspace(cfg.num_seqs, cfg.num_heads, cfg.head_dim, wl.max_context_len,
                                P, q.device) if P else None
    maxlen = wl.max_context_len
    has_copy = len(wl.block_mapping) > 0
    ev = []

    def decode():
        # With fused=True the decode launch also writes each sequence's newest K/V to its slot.
        if plan is not None:  # the groups and every other unit in one launch
            pk.paged_attention_decode_shared(q, kc, vc, bt, lens, groups, maxlen, cfg.scale, P,
                                             ws, work_items=order,
                                             new_key=key if fused else None,
                                             new_value=value if fused else None)
            return
        pk.paged_attention_decode(None if P else out, q, kc, vc, bt, lens, maxlen, cfg.scale,
                                  P, ws, kernel=kernel, work_items=order, cached_kv=cached,
                                  new_key=key if fused else None,
                                  new_value=value if fused else None)

    # When the step is the decode launch alone, one event pair brackets the whole timed region
    # and the mean launch duration is its span over the steps: events between the launches
    # would cost the loop time of their own (about 7 us per step on the GQA batch).
    alone = fused and not has_copy and not P

    def step(record):
        if has_copy:
            pk.copy_blocks([kc], [vc], mapping)
        if not fused:
            pk.reshape_and_cache(key, value, kc, vc, slots)
        if record and not alone:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        decode()
        if record and not alone:
            e1.record()
            ev.append((e0, e1))
        if P:
            pk.paged_attention_reduce(out, ws, lens, P)

    # Each kernel on its own, back to back (all of them are idempotent on these inputs). This
    # runs first: its ~0.1 s of sustained launches also brings the GPU out of idle before the
    # warm-up and timed steps.
    elt = 4 if cfg.dtype == "f32" else 2
    tile = cfg.num_kv_heads * cfg.block_size * cfg.head_dim * elt
    n_new = int((wl.slot_mapping >= 0).sum())
    kernels = {"paged_attention_decode": dict(
        launch_stats(torch, decode, args.launches, args.reps),
        kv_bytes=wl.kv_bytes())}
    kernels["reshape_and_cache"] = dict(
        launch_stats(torch, lambda: pk.reshape_and_cache(key, value, kc, vc, slots),
                     args.launches, args.reps),
        bytes=n_new * cfg.num_kv_heads * cfg.head_dim * elt * 2 * 2)
    if has_copy:
        kernels["copy_blocks"] = dict(
            launch_stats(torch, lambda: pk.copy_blocks([kc], [vc], mapping), args.launches,
                         args.reps),
            bytes=len(wl.block_mapping) * tile * 2 * 2)
    if P:
        kernels["paged_attention_reduce"] = dict(
            launch_stats(torch, lambda: pk.paged_attention_reduce(out, ws, lens, P),
                         args.launches, args.reps))
    for k, s in kernels.items():
        b = s.get("kv_bytes", s.get("bytes"))
        if b:
            s["GB_per_s"] = round(b / (s["median_us"] * 1e-6) / 1e9, 2)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    span[0].record()
    for _ in range(args.steps):
        step(True)
    span[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    if alone:
        dec_ms = span[0].elapsed_time(span[1]) / args.steps
    else:
        dec_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    print(f"[bench] {args.steps} steps, {ms_step:.4f} ms/step, decode {dec_ms:.4f} ms/launch",
          file=sys.stderr, flush=True)

    kvb = wl.kv_bytes()
    family = "mfma" if (kernel == "mfma" or (kernel == "auto" and cfg.dtype != "f32"
                                             and cfg.group >= 4)) else "valu"
    # The recorded counters belong to the workload as defined (its block size, whole batch).
    traffic = None if shard or cfg.block_size != W.CONFIGS[name].block_size \
        else counter_traffic(KERNEL_SOURCES[family], name, plan is not None)
    value = kvb / (ms_step * 1e-3) / 1e9
    ukvb = wl.unique_kv_bytes() if has_copy else kvb
    # With shared prefix blocks the logical bytes count the prefix once per sequence, but it is
    # served from cache after the first read: the HBM roofline takes the unique bytes.
    achieved = ukvb / (dec_ms * 1e-3) / 1e9
    line = {
        "metric": "paged decode KV-read GB/s (% of MI355X HBM peak) + attended tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{name}: {cfg.description}", "num_seqs": cfg.num_seqs,
                   "num_heads": cfg.num_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "block_size": cfg.block_size,
                   "num_blocks": cfg.num_blocks, "seed": cfg.seed,
                   "context_tokens": wl.total_tokens, "max_context_len": maxlen,
                   "kernel": kernel, "partition_size": P, "cached_kv": cached,
                   "shared_prefix": None if plan is None else {
                       "groups": len(plan.groups), "partition_size": P,
                       "members": int((plan.groups >= 0).sum())},
                   "fused_cache_write": fused, "kv_bytes": kvb,
                   "unique_kv_bytes": ukvb, "shard": shard},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "attended_tokens_per_s": round(wl.total_tokens / (ms_step * 1e-3), 1),
        "head_token_pairs_per_s": round(cfg.num_heads * wl.total_tokens / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": ("paged_attention_decode_shared (mfma: groups and other units)"
                                if plan is not None else f"paged_attention_decode ({family})"),
                     "ms_per_launch": round(dec_ms, 5), "bytes_per_launch": ukvb,
                     "logical_GB_per_s": round(kvb / (dec_ms * 1e-3) / 1e9, 2)},
        "kernels": kernels,
    }
    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30)) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n * 4
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
