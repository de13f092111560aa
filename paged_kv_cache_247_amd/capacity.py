"""Capacity and waste of KV-cache memory: the conventional contiguous reservation against
paged allocation, on the length distributions of the decode workloads.

    python -m paged_kv_cache_247_amd.capacity [--hbm-gib 288] [--weights-gib 16] [--layers 32]

The problem (Qualiteg, "About PagedAttention for LLM serving", "In a Nutshell ..." items 1-1
and 1-3, and the worked example under "Deepening Our Understanding of PagedAttention"): the
conventional engine reserves, per request and in advance, a contiguous KV region for the
maximum number of tokens the model handles, so a request that stops early wastes the rest
(the post's example: 1024 positions reserved, 13 generated, 1011 wasted). Sizing a server
that way gives (the same post, "Qualiteg classic hf-transformer" section):

    total memory = model weights + concurrent users * max context * KV bytes per token

Paged allocation (items 1-2 and 1-3) takes blocks of S positions as a sequence grows, so a
sequence holds ceil(L / S) * S positions and wastes at most S - 1 of them; the post puts the
useful block size at about 16 to 256 (larger blocks fragment again). Requests that share a
prefix share its blocks (Hacker News discussion of PagedAttention, replies on prefix sharing).

This is a host-side model; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import dataclasses

import numpy as np

from . import workload as W


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elt_bytes: int) -> int:
    """K and V of one position across all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elt_bytes


def contiguous_users(total_bytes: float, weight_bytes: float, max_context: int,
                     bytes_per_token: int) -> int:
    """Concurrent requests the contiguous reservation admits: the post's sizing formula solved
    for the number of users."""
    free = total_bytes - weight_bytes
    if free <= 0:
        return 0
    return int(free // (max_context * bytes_per_token))


def paged_positions(lens: np.ndarray, block_size: int) -> np.ndarray:
    """Positions each sequence holds under paging: whole blocks, ceil(L / S) * S."""
    L = np.asarray(lens, dtype=np.int64)
    return -(-L // block_size) * block_size


def shared_prefix_positions(lens: np.ndarray, prefix_len: int, block_size: int) -> int:
    """Positions a batch holds when all of its sequences share the first prefix_len positions:
    the prefix's blocks once (whole blocks only; a partial last prefix block is private), plus
    each sequence's own blocks after them."""
    L = np.asarray(lens, dtype=np.int64)
    shared_blocks = prefix_len // block_size
    own = -(-(L - shared_blocks * block_size) // block_size)
    return int(shared_blocks * block_size + (np.maximum(own, 0) * block_size).sum())


def waste_fraction(used: float, held: float) -> float:
    return 0.0 if held == 0 else 1.0 - used / held


def paged_users(lens_stream: np.ndarray, pool_positions: int, block_size: int) -> int:
    """Requests admitted in arrival order until the next one's blocks no longer fit."""
    need = np.cumsum(paged_positions(lens_stream, block_size))
    return int(np.searchsorted(need, pool_positions, side="right"))


@dataclasses.dataclass
class Row:
    workload: str
    block_size: int
    mean_len: float
    max_context: int
    contiguous_waste: float
    paged_waste: float
    paged_waste_shared: float | None
    contiguous_users: int
    paged_users: int
    paged_users_shared: int | None


def length_sample(cfg: W.Config, n: int, seed: int) -> np.ndarray:
    """n context lengths from the workload's own length distribution."""
    rng = np.random.default_rng(seed)
    return W.draw_lengths(cfg.replace(num_seqs=n), rng)


def model(names=("c2", "c3", "c4", "c5"), block_sizes=(16, 32, 64, 128, 256),
          hbm_gib: float = 288.0, weights_gib: float = 16.0, layers: int = 32,
          sample: int = 200_000, seed: int = 7) -> list[Row]:
    rows = []
    for name in names:
        cfg = W.CONFIGS[name]
        lens = length_sample(cfg, sample, seed)
        bpt = kv_bytes_per_token(layers, cfg.num_kv_heads, cfg.head_dim, W.elt_bytes(cfg.dtype))
        max_ctx = cfg.max_len
        total, weights = hbm_gib * 2 ** 30, weights_gib * 2 ** 30
        pool = int((total - weights) // bpt)
        c_users = contiguous_users(total, weights, max_ctx, bpt)
        used = float(lens.sum())
        for S in block_sizes:
            held = float(paged_positions(lens, S).sum())
            p_users = paged_users(lens, pool, S)
            shared = shared_users = None
            if cfg.len_dist == "prefix":
                distinct = cfg.prefix_len + float((lens - cfg.prefix_len).sum())
                shared = waste_fraction(distinct,
                                        shared_prefix_positions(lens, cfg.prefix_len, S))
                # admitted users when all of them share one prefix
                per_own = paged_positions(lens - (cfg.prefix_len // S) * S, S)
                room = pool - (cfg.prefix_len // S) * S
                shared_users = int(np.searchsorted(np.cumsum(per_own), room, side="right"))
            rows.append(Row(name, S, float(lens.mean()), max_ctx,
                            waste_fraction(used, len(lens) * float(max_ctx)),
                            waste_fraction(used, held), shared, c_users, p_users,
                            shared_users))
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--hbm-gib", type=float, default=288.0)
    ap.add_argument("--weights-gib", type=float, default=16.0)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--sample", type=int, default=200_000)
    args = ap.parse_args()
    rows = model(hbm_gib=args.hbm_gib, weights_gib=args.weights_gib, layers=args.layers,
                 sample=args.sample)
    print(f"KV budget: {args.hbm_gib:g} GiB HBM - {args.weights_gib:g} GiB weights; "
          f"{args.layers} layers; lengths: {args.sample} draws per workload")
    print("| workload | S | mean L | max ctx | contiguous waste | paged waste | "
          "users contiguous | users paged | x |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        pw = f"{100 * r.paged_waste:.2f}%"
        pu = f"{r.paged_users}"
        if r.paged_waste_shared is not None:
            pw += f" ({100 * r.paged_waste_shared:.2f}% shared)"
            pu += f" ({r.paged_users_shared} shared)"
        ratio = r.paged_users / max(r.contiguous_users, 1)
        print(f"| {r.workload} | {r.block_size} | {r.mean_len:.0f} | {r.max_context} | "
              f"{100 * r.contiguous_waste:.1f}% | {pw} | {r.contiguous_users} | {pu} | "
              f"{ratio:.2f} |")


if __name__ == "__main__":
    main()
