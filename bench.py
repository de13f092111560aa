"""Paged decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3] [--kernel auto]
                    [--partition-size P] [--unfused] [--layout paged] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch: copy-on-write block copies (when
the workload has them), the cache write of each sequence's newest token, paged decode, and the
partition merge when the context is split. By default the cache write is fused into the decode
launch (--unfused writes with a separate reshape_and_cache launch). Inputs are resident in HBM
before timing starts.

Prints one JSON line: KV-read GB/s over the step (value), attended tokens/s, the decode
kernel's roofline figures (timed per launch with HIP events on the launch stream), repetition
statistics of back-to-back launches of each kernel on its own (decode, cache write, block copy,
merge), the oracle's CPU throughput on the same workload at one thread and at all cores, and
the largest difference between the timed step's output and the oracle's over every sequence
(the run exits with status 3 if it is above tolerance). The default run (the grouped-query
batch) adds the other four workloads in their own launch configurations (`configs`), what the
block table costs against the contiguous reservation (`paging_cost`), and the read bandwidth
HBM gives a kernel that only loads (`read_ceiling`).

The oracle runs only in the CPU-baseline leg: its timed passes are over the step's own input
pools, and the last pass is the expected output. The main workload's oracle is timed first,
before anything touches the GPU, so its worker processes are plain CPU processes.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import platform
import sys
import time
from types import SimpleNamespace

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix-core peak, AMD published
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}  # max |gpu - oracle|, fp32 accumulation

# The pages' only figure on the kernel's speed; another machine's, quoted as context.
PAGES_CLAIM = {
    "claim": "a paged attention kernel was up to 2.85x slower than its FlashAttention "
             "counterpart for grouped-query attention",
    "source": "vAttention paper, section 3.1 (its Figure 9b, not reproduced on the page)",
    "hardware": "not stated on the page"}

# Launch configuration the benchmark uses for each workload: (kernel family, partition size,
# cached K/V loads). With longest-first dispatch, single-pass decode is fastest for the GQA
# batch (matrix-core workgroups fill two whole rounds of the GPU); the MHA batch's vector-ALU
# grid is 1.33 rounds, and 768-token partitions plus the merge even out its last round (step
# 183.4 against 185.9 us single pass, back to back); the lognormal long-context batch (up to
# ~31k tokens) splits into the 512-token partitions its statement names; the prefix-shared
# batch keeps K/V in cache so the shared prefix is reused.
LAUNCH = {
    "c1": ("auto", 0, False),
    "c2": ("auto", 768, False),
    "c3": ("auto", 0, False),
    "c4": ("auto", 0, True),
    "c5": ("auto", 512, False),
}
# The other workloads reported beside the default one: (workload, partition size override).
# The long-context batch also in 2048-token partitions (an option, not its stated launch).
CONFIG_BLOCK = [("c1", None), ("c2", None), ("c4", None), ("c5", None), ("c5", 2048)]

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
    ap.add_argument("--layout", default="paged",
                    help="paged (scattered blocks, block tables); contiguous (each sequence's "
                         "blocks in order, read without tables); contiguous-table (the same "
                         "layout read through identity tables); vmm:<page bytes> (the "
                         "contiguous layout in HIP virtual memory mapped in pages of that size)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (and with it the check of the output)")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run without the other workloads, the paging cost and the "
                         "read ceiling (the other workloads also need the oracle: they are "
                         "left out with --no-cpu-baseline)")
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
    ap.add_argument("--shared-prefix", default="auto", choices=["auto", "whole", "on", "off"],
                    help="decode blocks that sequences share once per group of sequences: "
                         "whole = one pass per group over the shared and its members' own "
                         "positions; on = the groups' shared partition beside the other "
                         "split-context units, then the merge; auto = whole when every "
                         "sequence can join a group, else on, when the batch shares a prefix "
                         "and runs single pass; off = plain decode")
    ap.add_argument("--block-size", type=int, default=None,
                    help="run the workload in blocks of this many positions (16..256); the "
                         "pool keeps at least its capacity")
    ap.add_argument("--shard", default=None, metavar="KIND:N",
                    help="run one GPU's share of an N-GPU job at its real shape: kv:N keeps "
                         "1/N of the kv heads (and their q heads), seq:N 1/N of the sequences")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    ap.add_argument("--between-launches", default=None, choices=list(BETWEEN),
                    help="also time single decode launches (an event pair around each, a "
                         "synchronisation between them) with nothing before each and with this "
                         "work before each: l2 = a copy moving 32 MiB (the L2s), llc = a copy "
                         "moving 1 GiB (also the last-level cache and many page translations), "
                         "tlb = one byte read per 64 KiB of 8 GiB (page translations, little "
                         "data)")
    args = ap.parse_args()
    layout = args.layout
    if not (layout in ("paged", "contiguous", "contiguous-table") or
            (layout.startswith("vmm:") and layout[4:].isdigit())):
        ap.error(f"--layout {layout}: expected paged, contiguous, contiguous-table or "
                 "vmm:<page bytes>")
    return args


# ------------------------------------------------------------------ oracle on the CPU

_POOLS = None  # (workload, k pool, v pool) of the step, inherited by forked oracle workers


def step_pools(wl):
    """The pools one step decodes over: the copy-on-write copies and the newest tokens' cache
    writes applied by the oracle (untimed: this is the step's input, not its decode)."""
    import oracle
    c = wl.cfg
    kc, vc = oracle.write_cache(wl.k_cache, wl.v_cache, wl.key, wl.value, wl.slot_mapping,
                                c.block_size)
    if len(wl.block_mapping):
        (kc,), (vc,) = oracle.copy_blocks([kc], [vc], wl.block_mapping)
    return kc, vc


def _oracle_decode(wl, kc, vc, idx=None):
    import oracle
    c = wl.cfg
    if idx is None:
        return oracle.decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, c.scale,
                             c.num_kv_heads, c.dtype)
    return oracle.decode(wl.q[idx], kc, vc, wl.block_tables[idx], wl.context_lens[idx],
                         c.scale, c.num_kv_heads, c.dtype)


def _oracle_part(idx):
    """One worker's share of an oracle pass: decode of the sequences idx on one thread."""
    from threadpoolctl import threadpool_limits
    wl, kc, vc = _POOLS
    with threadpool_limits(limits=1):
        _oracle_decode(wl, kc, vc, idx)
    return int(wl.context_lens[idx].sum())


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
    """The oracle's decode (fp64 numpy) over whole passes of the step's pools: first on one
    thread for about one_s seconds (at least one pass), then split over `workers` forked
    processes (one thread each) for about all_s seconds of wall time. Returns the figures and
    the last one-thread pass's output (the expected output of the step)."""
    global _POOLS
    from threadpoolctl import threadpool_limits
    c = wl.cfg
    kc, vc = step_pools(wl)
    per_tok = c.num_kv_heads * c.head_dim * (4 if c.dtype == "f32" else 2) * 2
    passes, toks, dt = 0, 0, 0.0
    expected = None
    with threadpool_limits(limits=1):
        while passes == 0 or dt < one_s:
            t0 = time.perf_counter()
            expected = _oracle_decode(wl, kc, vc)
            dt += time.perf_counter() - t0
            passes += 1
            toks += wl.total_tokens
    what = "pass" if passes == 1 else "passes"
    res = {"value": round(toks * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"{passes} whole {what} over all {c.num_seqs} sequences ({wl.total_tokens} "
                     f"context tokens each), fp64 numpy decode on one thread, {dt:.1f} s",
           "attended_tokens_per_s": round(toks / dt, 1),
           "cpu": cpu_model(), "host_cpus": os.cpu_count()}
    if workers > 1 and all_s > 0:
        _POOLS = (wl, kc, vc)
        shares = _shares(wl.context_lens, workers)
        with mp.get_context("fork").Pool(len(shares)) as pool:
            pool.map(_oracle_part, shares)  # start-up and first touch, untimed
            passes, toks = 0, 0
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < all_s:
                toks += sum(pool.map(_oracle_part, shares))
                passes += 1
            dt = time.perf_counter() - t0
        _POOLS = None
        res["all_cores"] = {
            "value": round(toks * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": len(shares),
            "sample": f"{passes} whole passes split over {len(shares)} processes (one thread "
                      f"each, sequences balanced by length), {dt:.1f} s wall",
            "attended_tokens_per_s": round(toks / dt, 1)}
    return res, expected


def parity(out, expected, dtype: str, what: str) -> dict:
    """Largest |gpu - oracle| over every element of the step's output."""
    got = out.detach().float().cpu().numpy().astype(np.float64)
    d = np.abs(got - expected)
    err = float("inf") if np.isnan(d).any() else float(d.max()) if d.size else 0.0
    return {"max_abs_err": err, "tol": TOL[dtype], "ok": bool(err <= TOL[dtype]),
            "compared": what, "oracle": "fp64 numpy, the cpu_baseline leg's last pass"}


# ------------------------------------------------------------------ GPU helpers

def counter_traffic(kernel_sources, workload, shared=False, partition_size=0):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if the summary
    was taken on the kernel sources as they are now and in the same decode mode (the grouped
    shared-prefix launches or not, the same partition size), else None."""
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
    if vals.get("shared_prefix", "0") != str(shared if isinstance(shared, str) else int(bool(shared))):
        return None
    if vals.get("partition_size", "0") != str(int(partition_size)):
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


# Work run before each launch by --between-launches: what a layer's decode finds in the memory
# system when other work ran since its previous launch.
BETWEEN = {"l2": "device copy of 16 MiB (32 MiB moved)",
           "llc": "device copy of 512 MiB (1 GiB moved)",
           "tlb": "one byte read per 64 KiB of an 8 GiB buffer"}


def between_launches(torch, fn, mode: str, rounds: int = 3, launches: int = 20):
    """Microseconds per single launch of fn (an event pair around it, a synchronisation after
    it), medians over `launches` for each of `rounds` rounds, without and with the work named
    by `mode` before each launch."""
    if mode == "tlb":
        buf = torch.zeros(8 << 30, dtype=torch.uint8, device="cuda").view(-1, 65536)
        before = lambda: buf[:, 0].sum()  # noqa: E731
    else:
        n = (32 << 20) if mode == "l2" else (1 << 30)
        a = torch.zeros(n // 2, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        before = lambda: b.copy_(a)  # noqa: E731
    res = {"nothing": [], mode: []}
    for _ in range(rounds):
        for key in res:
            ts = []
            for _ in range(launches):
                if key != "nothing":
                    before()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            ts.sort()
            res[key].append(round(ts[len(ts) // 2], 2))
    return {"before_each_launch": BETWEEN[mode], "us_with_nothing_before": res["nothing"],
            "us_with_it_before": res[mode], "rounds": rounds, "launches_per_round": launches}


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


def kernel_family(kernel, cfg, table_free=False):
    if kernel == "mfma" or table_free:
        return "mfma"
    if kernel == "auto" and cfg.dtype != "f32" and cfg.group >= 4:
        return "mfma"
    return "valu"


def build_step(torch, pk, wl, kernel, P, cached, shared_prefix="auto", fused=True,
               layout="paged"):
    """Device copies of a workload and the closures of one decode step.

    layout "paged" decodes through the block tables; "contiguous" and "vmm:<bytes>" expect the
    contiguous layout (workload.contiguous_layout) and decode without tables, the latter from a
    virtual-memory pool; "contiguous-table" reads the contiguous layout through its identity
    tables."""
    cfg = wl.cfg
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def dev(a, bf=cfg.dtype == "bf16"):
        a = np.ascontiguousarray(a)
        if bf:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    s = SimpleNamespace(cfg=cfg, wl=wl, kernel=kernel, P=P, cached=cached, fused=fused,
                        layout=layout, plan=None, whole=None, pool=None)
    s.q, s.key, s.value = dev(wl.q), dev(wl.key), dev(wl.value)
    s.kc, s.vc = dev(wl.k_cache), dev(wl.v_cache)
    s.slots = dev(wl.slot_mapping, False)
    s.bt, s.lens = dev(wl.block_tables, False), dev(wl.context_lens, False)
    s.mapping = dev(wl.block_mapping.reshape(-1, 2), False)
    table_free = layout == "contiguous" or layout.startswith("vmm:")
    MB = wl.block_tables.shape[1]
    if table_free:
        s.kernel = kernel = "mfma"  # the table-free reservation runs on the matrix-core kernel
        if not fused:
            raise ValueError("the table-free layouts take the fused newest-token write")
    if layout.startswith("vmm:"):
        s.pool = pk.VmmPool(cfg.num_seqs, wl.max_context_len, cfg.num_kv_heads, cfg.head_dim,
                            cfg.block_size, dt, page_bytes=int(layout[4:]))
        for i in range(cfg.num_seqs):
            L = int(wl.context_lens[i])
            nb = -(-L // cfg.block_size)
            s.pool.map(i, L)
            if nb:
                s.pool.write(i, s.kc[i * MB:i * MB + nb], s.vc[i * MB:i * MB + nb])
        torch.cuda.synchronize()
        s.kc = s.vc = None
        torch.cuda.empty_cache()
        kpool, vpool, MB = s.pool.k, s.pool.v, s.pool.blocks_per_seq
    else:
        kpool, vpool = s.kc, s.vc
    s.family = kernel_family(kernel, cfg, table_free)
    # Blocks shared by several sequences (a common prefix): plan groups that read each shared
    # tile once for all their members (host scheduler input, like the work list).
    from paged_kv_cache_247_amd import sharing
    if shared_prefix == "whole" or (shared_prefix == "auto" and cfg.prefix_len and not P):
        s.whole = sharing.plan_whole(wl.block_tables, wl.context_lens, cfg.block_size,
                                     cfg.group, newest_outside=fused)
        if s.whole is None and shared_prefix == "whole":
            raise ValueError("--shared-prefix whole: no blocks are shared, or a sequence is too "
                             "short to join a group")
    if s.whole is None and (shared_prefix == "on" or
                            (shared_prefix == "auto" and cfg.prefix_len and not P)):
        s.plan = sharing.plan(wl.block_tables, wl.context_lens, cfg.block_size,
                              wl.max_context_len, cfg.group, newest_outside=fused)
        if s.plan is None and shared_prefix == "on":
            raise ValueError("--shared-prefix on: no blocks are shared")
    if s.whole is not None:
        s.P, s.kernel, s.cached, s.family = 0, "mfma", True, "mfma"
        s.groups = dev(s.whole.groups, False)
        s.order = None
    elif s.plan is not None:
        s.P, s.kernel, s.cached, s.family = s.plan.partition_size, "mfma", True, "mfma"
        s.groups = dev(s.plan.groups, False)
        s.order = dev(s.plan.work_items, False)
    else:
        # Host-side scheduler input: the units with work, largest first.
        s.order = dev(wl.work_items(P), False)
    P = s.P
    s.out = torch.empty((cfg.num_seqs, cfg.num_heads, cfg.head_dim), dtype=dt, device="cuda")
    s.ws = pk.partition_workspace(cfg.num_seqs, cfg.num_heads, cfg.head_dim,
                                  wl.max_context_len, P, s.q.device) if P else None
    s.has_copy = len(wl.block_mapping) > 0
    maxlen = wl.max_context_len
    nk, nv = (s.key, s.value) if fused else (None, None)
    bt = None if table_free else s.bt

    def decode():
        # With fused=True the decode launch also writes each sequence's newest K/V to its slot.
        if s.whole is not None:  # one pass per group, shared and own positions
            pk.paged_attention_decode_grouped(s.out, s.q, kpool, vpool, s.bt, s.lens, s.groups,
                                              s.whole.shared_len, cfg.scale, new_key=nk,
                                              new_value=nv)
            return
        if s.plan is not None:  # the groups and every other unit in one launch
            pk.paged_attention_decode_shared(s.q, kpool, vpool, s.bt, s.lens, s.groups, maxlen,
                                             cfg.scale, P, s.ws, work_items=s.order,
                                             new_key=nk, new_value=nv)
            return
        pk.paged_attention_decode(None if P else s.out, s.q, kpool, vpool, bt, s.lens, maxlen,
                                  cfg.scale, P, s.ws, kernel=s.kernel, work_items=s.order,
                                  cached_kv=s.cached, new_key=nk, new_value=nv,
                                  max_blocks_per_seq=MB if table_free else None)

    def reduce():
        pk.paged_attention_reduce(s.out, s.ws, s.lens, P)

    def step(events=None):
        if s.has_copy:
            pk.copy_blocks([kpool], [vpool], s.mapping)
        if not fused:
            pk.reshape_and_cache(s.key, s.value, kpool, vpool, s.slots)
        if events is not None:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        decode()
        if events is not None:
            e1.record()
            events.append((e0, e1))
        if P:
            reduce()

    def release():
        if s.pool is not None:
            s.pool.close()
        for k in ("q", "key", "value", "kc", "vc", "slots", "bt", "lens", "mapping", "out",
                  "ws", "order", "groups"):
            setattr(s, k, None)
        torch.cuda.empty_cache()

    s.decode, s.reduce, s.step, s.release = decode, reduce, step, release
    s.kpool, s.vpool = kpool, vpool
    return s


def kernel_name(s):
    if s.whole is not None:
        return "paged_attention_decode_grouped (mfma: whole groups over a shared prefix)"
    if s.plan is not None:
        return "paged_attention_decode_shared (mfma: groups and other units)"
    return f"paged_attention_decode ({s.family})"


def roofline_bytes(wl):
    """Bytes the decode launch must read: the KV bytes, or with shared blocks the distinct
    tiles (the shared prefix is served from cache after its first read), without the
    copy-on-write copies (a launch of their own)."""
    return wl.unique_kv_bytes(include_copies=False) if len(wl.block_mapping) or \
        wl.cfg.prefix_len else wl.kv_bytes()


def config_entry(torch, pk, name, P_over, reps, launches):
    """One workload in its own launch configuration: step and decode-launch timing, the
    roofline fraction, the output against the oracle and a one-pass CPU baseline."""
    from paged_kv_cache_247_amd import workload as W
    kernel, P, cached = LAUNCH[name]
    P = P if P_over is None else P_over
    cfg = W.CONFIGS[name]
    t0 = time.time()
    wl = W.generate(cfg, poison="zero")
    cpu, expected = cpu_baseline(wl, 0.0, 0.0, 1)
    print(f"[bench] {name} P={P}: generated and oracle in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    s = build_step(torch, pk, wl, kernel, P, cached)
    dec = launch_stats(torch, s.decode, launches, reps)
    stp = launch_stats(torch, s.step, launches, reps)
    s.step()
    torch.cuda.synchronize()
    chk = parity(s.out, expected, cfg.dtype,
                 f"all {cfg.num_seqs} sequences x {cfg.num_heads} heads x {cfg.head_dim}")
    kvb, rb = wl.kv_bytes(), roofline_bytes(wl)
    entry = {
        "workload": f"{name}: {cfg.description}", "seed": cfg.seed,
        "context_tokens": wl.total_tokens, "kv_bytes": kvb,
        "kernel": kernel_name(s),
        "partition_size": s.P, "cached_kv": s.cached,
        "step_us": stp["median_us"],
        "GB_per_s": round(kvb / (stp["median_us"] * 1e-6) / 1e9, 2),
        "attended_tokens_per_s": round(wl.total_tokens / (stp["median_us"] * 1e-6), 1),
        "decode_us": dec["median_us"],
        "roofline": {"bound": "hbm", "bytes_per_launch": rb,
                     "achieved": round(rb / (dec["median_us"] * 1e-6) / 1e9, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(rb / (dec["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
        "max_abs_err": chk["max_abs_err"], "tol": chk["tol"], "parity_ok": chk["ok"],
        "cpu_baseline": {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
    }
    if P_over is not None:
        entry["note"] = f"partition size {P} is an option; the workload states {LAUNCH[name][1]}"
    s.release()
    return entry


def paging_cost(torch, pk, wl, paged_us, paged_out, reps, launches):
    """The same batch, kernel and work list in the conventional contiguous reservation read
    without block tables: what the block table costs the decode launch here."""
    from paged_kv_cache_247_amd import workload as W
    kernel, P, cached = LAUNCH[wl.cfg.name] if wl.cfg.name in LAUNCH else ("auto", 0, False)
    wc = W.contiguous_layout(wl)
    s = build_step(torch, pk, wc, kernel, P, cached, layout="contiguous")
    st = launch_stats(torch, s.decode, launches, reps)
    s.step()
    torch.cuda.synchronize()
    same = bool(torch.equal(s.out.view(torch.uint8), paged_out.view(torch.uint8)))
    s.release()
    return {"paged_us": paged_us, "contiguous_no_table_us": st["median_us"],
            "paged_over_contiguous": round(paged_us / st["median_us"], 4),
            "outputs_bit_identical": same,
            "what": "decode launch, median of back-to-back launches; same kernel, inputs and "
                    "work list, blocks scattered through the pool and read through block "
                    "tables against each sequence's blocks in order read without them "
                    "(bench.py --layout contiguous|vmm:<page bytes> runs either as the step)",
            "pages_context": PAGES_CLAIM}


def read_ceiling(torch, pk, wl, reps, launches, seed=7):
    """What HBM delivers to kernels that only load: one streaming read of a buffer the size of
    the workload's two pools, and random gathers of whole tiles -- the (block, kv head) tiles
    decode reads (S * D * elt bytes), in random order -- and of 8 KiB tiles."""
    c = wl.cfg
    elt = 4 if c.dtype == "f32" else 2
    tile = c.block_size * c.head_dim * elt
    pool_bytes = c.num_blocks * c.num_kv_heads * tile
    total = (2 * pool_bytes) // 32768 * 32768
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {"buffer_bytes": total}

    def gbps(nbytes, us):
        return round(nbytes / (us * 1e-6) / 1e9, 2)

    for nt in (True, False):
        st = launch_stats(torch, lambda: pk.probe_stream_read(buf, sink, nontemporal=nt),
                          launches, reps, warmup=3)
        res[f"stream{'_nt' if nt else ''}_GB_per_s"] = gbps(total, st["median_us"])
    rng = np.random.default_rng(seed)
    if tile in (4096, 8192):
        # the tiles decode reads: K and V of every used (block, kv head), in random order
        S = c.block_size
        offs = []
        for i, L in enumerate(wl.context_lens):
            nb = -(-int(L) // S)
            b = wl.block_tables[i, :nb].astype(np.int64)
            t = (b[:, None] * c.num_kv_heads + np.arange(c.num_kv_heads)[None, :]).ravel()
            offs.append(t * tile)
            offs.append(pool_bytes + t * tile)
        offs = np.concatenate(offs)
        offs = offs[rng.permutation(len(offs))]
        n_bytes = len(offs) * tile
        d_offs = torch.from_numpy(offs).cuda()
        for nt in (True, False):
            st = launch_stats(torch, lambda: pk.probe_tile_gather(buf, d_offs, tile, sink,
                                                                  nontemporal=nt),
                              launches, reps, warmup=3)
            res[f"gather_{tile // 1024}KiB{'_nt' if nt else ''}_GB_per_s"] = \
                gbps(n_bytes, st["median_us"])
        res["gather_tiles"] = len(offs)
    # 8 KiB tiles at random distinct 8 KiB-aligned places, the same number of bytes
    n8 = max(1, min(total // 8192, (len(offs) * tile if tile in (4096, 8192) else total // 2)
                    // 8192))
    offs8 = rng.choice(total // 8192, size=n8, replace=False).astype(np.int64) * 8192
    d8 = torch.from_numpy(offs8).cuda()
    st = launch_stats(torch, lambda: pk.probe_tile_gather(buf, d8, 8192, sink, nontemporal=True),
                      launches, reps, warmup=3)
    res["gather_8KiB_random_nt_GB_per_s"] = gbps(n8 * 8192, st["median_us"])
    del buf, d8
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ prefill

def prefill_cpu_baseline(wl, one_s: float):
    """The prefill oracle (fp64 numpy, one thread) over whole sequences of the workload,
    longest contexts first, until about one_s seconds have run. Returns the figures and the
    expected output rows of the sequences it ran."""
    from threadpoolctl import threadpool_limits

    import oracle
    c = wl.cfg
    done, flops, dt = 0, 0, 0.0
    expected = {}
    with threadpool_limits(limits=1):
        for i in np.argsort(-wl.context_lens, kind="stable"):
            if dt >= one_s:
                break
            L, Q = int(wl.context_lens[i]), int(wl.query_lens[i])
            r0 = int(wl.query_start[i])
            t0 = time.perf_counter()
            expected[int(i)] = oracle.prefill(
                wl.q_prefill[r0:r0 + Q], wl.k_cache, wl.v_cache, wl.block_tables[i:i + 1],
                wl.context_lens[i:i + 1], np.array([0, Q], dtype=np.int32), c.scale,
                c.num_kv_heads, c.dtype)
            dt += time.perf_counter() - t0
            done += 1
            flops += (2 * (L - Q) + Q + 1) * Q // 2 * c.num_heads * c.head_dim * 4
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {c.num_seqs} sequences (longest contexts first), fp64 numpy "
                      f"prefill on one thread, {dt:.1f} s",
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}, expected


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
    cpu, expected = (None, None) if args.no_cpu_baseline else \
        prefill_cpu_baseline(wl, args.cpu_seconds)
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

    # The chunk's own cache write: its new tokens' K/V rows (already in the pool, so rewriting
    # them is idempotent) at the slots of positions L - Q .. L - 1, consecutive runs per block.
    S = cfg.block_size
    slots = np.concatenate([
        wl.block_tables[i, np.arange(L - Q, L) // S].astype(np.int64) * S + np.arange(L - Q, L) % S
        for i, (L, Q) in enumerate(zip(wl.context_lens.astype(np.int64),
                                       wl.query_lens.astype(np.int64)))])
    pos_rows = [(i, p) for i, (L, Q) in enumerate(zip(wl.context_lens, wl.query_lens))
                for p in range(int(L - Q), int(L))]
    knew = np.stack([wl.k_cache[wl.block_tables[i, p // S], :, p % S, :] for i, p in pos_rows])
    VS = min(S, 32)
    vv = wl.v_cache.reshape(wl.v_cache.shape[0], cfg.num_kv_heads, S // VS, cfg.head_dim, VS)
    vnew = np.stack([vv[wl.block_tables[i, p // S], :, (p % S) // VS, :, p % VS]
                     for i, p in pos_rows])
    dkey, dval, dslots = dev(knew), dev(vnew), dev(slots)

    kernels = {"paged_attention_prefill": launch_stats(torch, prefill, args.launches, args.reps)}
    kernels["reshape_and_cache"] = dict(
        launch_stats(torch, lambda: pk.reshape_and_cache(dkey, dval, kc, vc, dslots),
                     args.launches, args.reps),
        bytes=2 * 2 * int(knew.nbytes), tokens=len(slots))
    kernels["reshape_and_cache"]["GB_per_s"] = round(
        kernels["reshape_and_cache"]["bytes"] / (kernels["reshape_and_cache"]["median_us"] * 1e-6)
        / 1e9, 2)
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
    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30)) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n * 4
    ok = True
    if cpu is not None:
        line["cpu_baseline"] = cpu
        got = out.float().cpu().numpy().astype(np.float64)
        err = 0.0
        for i, ref in expected.items():
            r0, Q = int(wl.query_start[i]), int(wl.query_lens[i])
            d = np.abs(got[r0:r0 + Q] - ref)
            err = max(err, float("inf") if np.isnan(d).any() else float(d.max()))
        ok = err <= TOL[cfg.dtype]
        line["parity"] = {"max_abs_err": err, "tol": TOL[cfg.dtype], "ok": bool(ok),
                          "compared": f"every query row of the {len(expected)} sequences the "
                                      "cpu_baseline leg ran",
                          "oracle": "fp64 numpy, the cpu_baseline leg"}
    print(json.dumps(line), flush=True)
    if not ok:
        print("[bench] output differs from the oracle beyond tolerance", file=sys.stderr)
        sys.exit(3)


# ------------------------------------------------------------------ decode

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
        n = int(n) if n.isdigit() else 0
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
    if args.layout != "paged" and (cfg.prefix_len or args.unfused):
        print(f"--layout {args.layout}: the contiguous layouts hold no shared blocks and take "
              "the fused cache write", file=sys.stderr)
        sys.exit(2)
    t0 = time.time()
    wl = W.generate(cfg, poison="zero")
    if args.layout != "paged":
        wl = W.contiguous_layout(wl)
    print(f"[bench] generated {name} ({args.layout}) in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)

    cpu = expected = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        print(f"[bench] timing the oracle on the CPU (1 thread, then {workers} processes)",
              file=sys.stderr, flush=True)
        cpu, expected = cpu_baseline(wl, args.cpu_seconds, args.cpu_all_seconds, workers)

    import torch

    import paged_kv_cache_247_amd as pk
    pk.load()  # fails loudly when the library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    fused = not args.unfused
    try:
        s = build_step(torch, pk, wl, kernel, P, cached, args.shared_prefix, fused, args.layout)
    except ValueError as e:
        print(str(e), file=sys.stderr)
        sys.exit(2)
    P, kernel, cached = s.P, s.kernel, s.cached
    maxlen = wl.max_context_len
    # When the step is the decode launch alone, one event pair brackets the whole timed region
    # and the mean launch duration is its span over the steps: events between the launches
    # would cost the loop time of their own (about 7 us per step on the GQA batch).
    alone = fused and not s.has_copy and not P
    ev = []

    # Each kernel on its own, back to back (all of them are idempotent on these inputs). This
    # runs first: its ~0.1 s of sustained launches also brings the GPU out of idle before the
    # warm-up and timed steps.
    elt = 4 if cfg.dtype == "f32" else 2
    tile = cfg.num_kv_heads * cfg.block_size * cfg.head_dim * elt
    n_new = int((wl.slot_mapping >= 0).sum())
    kernels = {"paged_attention_decode": dict(
        launch_stats(torch, s.decode, args.launches, args.reps), kv_bytes=wl.kv_bytes())}
    if args.layout == "paged":
        kernels["reshape_and_cache"] = dict(
            launch_stats(torch, lambda: pk.reshape_and_cache(s.key, s.value, s.kc, s.vc,
                                                             s.slots),
                         args.launches, args.reps),
            bytes=n_new * cfg.num_kv_heads * cfg.head_dim * elt * 2 * 2)
    if s.has_copy:
        kernels["copy_blocks"] = dict(
            launch_stats(torch, lambda: pk.copy_blocks([s.kc], [s.vc], s.mapping),
                         args.launches, args.reps),
            bytes=len(wl.block_mapping) * tile * 2 * 2)
    if P:
        kernels["paged_attention_reduce"] = dict(
            launch_stats(torch, s.reduce, args.launches, args.reps))
    for k, st in kernels.items():
        b = st.get("kv_bytes", st.get("bytes"))
        if b:
            st["GB_per_s"] = round(b / (st["median_us"] * 1e-6) / 1e9, 2)

    for _ in range(args.warmup):
        s.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    span[0].record()
    for _ in range(args.steps):
        s.step()
    span[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    in_step_ms = None
    if alone:
        dec_ms = span[0].elapsed_time(span[1]) / args.steps
    else:
        # The step has other kernels too. The timed steps above hold no events: an event pair
        # around each decode launch opens gaps of its own (a few us per step), which would be
        # charged to the step. The launch duration is taken the way it is for a step of the
        # decode alone -- the same launch repeated `steps` times back to back under one event
        # pair (its inputs are unchanged by a repeat) -- and a further `steps` steps with an
        # event pair around each decode give the in-step figure reported beside it.
        for _ in range(args.steps):
            s.step(ev)
        torch.cuda.synchronize()
        in_step_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            s.decode()
        e1.record()
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps, {ms_step:.4f} ms/step, decode {dec_ms:.4f} ms/launch",
          file=sys.stderr, flush=True)
    check = None
    if expected is not None:
        check = parity(s.out, expected, cfg.dtype,
                       f"the timed step's output, all {cfg.num_seqs} sequences x "
                       f"{cfg.num_heads} heads x {cfg.head_dim}")
        print(f"[bench] max abs err against the oracle {check['max_abs_err']:.3g} "
              f"(tolerance {check['tol']})", file=sys.stderr, flush=True)

    kvb = wl.kv_bytes()
    # The recorded counters belong to the workload as defined (its block size, whole batch,
    # paged layout).
    traffic = None if shard or args.layout != "paged" or \
        cfg.block_size != W.CONFIGS[name].block_size \
        else counter_traffic(KERNEL_SOURCES[s.family], name,
                             "whole" if s.whole is not None else s.plan is not None, s.P)
    value = kvb / (ms_step * 1e-3) / 1e9
    rb = roofline_bytes(wl)
    # With shared prefix blocks the logical bytes count the prefix once per sequence, but it is
    # served from cache after the first read: the HBM roofline takes the unique bytes (without
    # the copy-on-write copies, which are a launch of their own).
    achieved = rb / (dec_ms * 1e-3) / 1e9
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
                   "layout": args.layout,
                   "shared_prefix": (
                       {"mode": "whole groups", "groups": len(s.whole.groups),
                        "shared_len": s.whole.shared_len,
                        "members": int((s.whole.groups >= 0).sum())} if s.whole is not None
                       else None if s.plan is None else
                       {"mode": "groups beside split-context units", "groups": len(s.plan.groups),
                        "partition_size": P, "members": int((s.plan.groups >= 0).sum())}),
                   "fused_cache_write": fused, "kv_bytes": kvb,
                   "unique_kv_bytes": wl.unique_kv_bytes(), "shard": shard},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "attended_tokens_per_s": round(wl.total_tokens / (ms_step * 1e-3), 1),
        "head_token_pairs_per_s": round(cfg.num_heads * wl.total_tokens / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": kernel_name(s),
                     "ms_per_launch": round(dec_ms, 5), "bytes_per_launch": rb,
                     "ms_per_launch_between_events_in_step": None if in_step_ms is None
                     else round(in_step_ms, 5),
                     "logical_GB_per_s": round(kvb / (dec_ms * 1e-3) / 1e9, 2)},
        "kernels": kernels,
        "parity": check,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if args.between_launches:
        print(f"[bench] single launches, {BETWEEN[args.between_launches]} before each",
              file=sys.stderr, flush=True)
        line["between_launches"] = between_launches(torch, s.decode, args.between_launches)

    default_run = (name == "c3" and args.layout == "paged" and not shard and not args.unfused
                   and args.block_size in (None, W.CONFIGS[name].block_size)
                   and args.kernel is None and args.partition_size is None)
    if default_run and not args.no_extras:
        paged_out = s.out.clone()
        paged_us = kernels["paged_attention_decode"]["median_us"]
        s.release()
        reps, launches = 3, 50
        print("[bench] read ceiling", file=sys.stderr, flush=True)
        ceil = read_ceiling(torch, pk, wl, reps, 20)
        g = ceil.get("gather_4KiB_nt_GB_per_s")
        ceil["decode_frac_of_gather_ceiling"] = round(achieved / g, 4) if g else None
        ceil["decode_frac_of_stream_ceiling"] = round(achieved / ceil["stream_nt_GB_per_s"], 4)
        line["read_ceiling"] = ceil
        print("[bench] paging cost", file=sys.stderr, flush=True)
        line["paging_cost"] = paging_cost(torch, pk, wl, paged_us, paged_out, reps, launches)
        del paged_out
        wl = None
        if not args.no_cpu_baseline:  # each workload's output is checked against the oracle
            line["configs"] = {}
            for cname, p_over in CONFIG_BLOCK:
                key = cname if p_over is None else f"{cname}_p{p_over}"
                line["configs"][key] = config_entry(torch, pk, cname, p_over, reps, launches)
            line["configs"]["c3"] = "the headline figures of this line"
    else:
        s.release()
    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30)) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n * 4
    print(json.dumps(line), flush=True)
    bad = [k for k, e in line.get("configs", {}).items()
           if isinstance(e, dict) and not e["parity_ok"]]
    if (check is not None and not check["ok"]) or bad:
        print(f"[bench] output differs from the oracle beyond tolerance "
              f"({'main' if check is not None and not check['ok'] else ''} {' '.join(bad)})",
              file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
