"""Seeded synthetic inputs for paged decode.

This module is the only code that both the oracle side and the HIP side use. It draws
context lengths, a scattered physical block pool, per-sequence block tables, the slot
mapping of each sequence's newest token and the copy-on-write choices of a shared prefix.
It holds none of the attention arithmetic: it only places a seeded logical K/V stream
into the pool layout that the C-ABI header documents.

Sources for what is generated:
  * KV cache split into fixed-size blocks that need not be contiguous, linked to each
    sequence through a table of logical-to-physical blocks; block sizes of 16..256 are the
    recommended range (Qualiteg, "About PagedAttention for LLM serving", sections
    "Deepening Our Understanding of PagedAttention" item 1-2 and "There are logical blocks
    and physical blocks, and the two are linked by a block table").
  * A ragged batch with no padding ("In a Nutshell ..." item 2-1 of the same post).
  * Requests that share a prompt prefix share its KV cache (Hacker News discussion of
    PagedAttention, replies on prefix sharing).

Pool layout (one layer):
  k_cache[N, Hkv, S, D]  -- token rows, head_dim contiguous
  v_cache[N, Hkv, (S/VS) D, VS], VS = min(S, 32) -- column groups of VS block positions,
      head_dim rows within each (position t, dim d at row (t // VS) D + d, column t % VS);
      for S <= 32 simply [N, Hkv, D, S]
bf16 values are carried as uint16 bit patterns (numpy has no bf16 type).

Reading of the length of a step: context_lens[i] counts the token written this step. The
pool holds logical positions 0..L_i-2 before the step; position L_i-1 arrives as
key/value rows plus a slot in slot_mapping.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# NaN bit patterns used to poison pool slots that no sequence owns.
_NAN_BITS = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def storage_dtype(dtype: str):
    """numpy type that holds one element of `dtype` (bf16 as its raw 16 bits)."""
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def elt_bytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns the uint16 bit patterns.

    Finite inputs only (the generator draws N(0,1) values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def v_group(block_size: int) -> int:
    """Positions per column group of the V pool layout."""
    return min(int(block_size), 32)


def v_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int):
    VS = v_group(block_size)
    return (num_blocks, num_kv_heads, block_size // VS * head_dim, VS)


def cast_from_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)  # numpy rounds to nearest even
    return bf16_bits_from_f32(x)


@dataclass(frozen=True)
class Config:
    """One synthetic paged-decode workload."""

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    seed: int
    len_dist: str  # "fixed" | "uniform" | "lognormal" | "prefix"
    lens: tuple = ()  # "fixed": the lengths themselves
    len_lo: int = 0  # "uniform"/"prefix": inclusive bounds (of the suffix for "prefix");
    len_hi: int = 0  # "lognormal": clip bounds
    lognormal_median: float = 0.0
    lognormal_sigma: float = 1.0
    prefix_len: int = 0  # "prefix": shared prefix tokens (a multiple of block_size)
    cow_seqs: int = 0  # "prefix": sequences whose last shared block gets a private copy
    partition_size: int = 0  # 0 = single pass; >0 = split-context partitions of this size
    # Query tokens per sequence: 0 = decode (the newest token only); > 0 = chunked prefill of
    # min(query_len, L_i) new tokens at the end of each context; -1 = whole-prompt prefill.
    query_len: int = 0
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_len(self) -> int:
        """Largest context length the length distribution can produce."""
        if self.len_dist == "fixed":
            return max(self.lens)
        if self.len_dist == "prefix":
            return self.prefix_len + self.len_hi
        return self.len_hi

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def with_block_size(self, S: int) -> "Config":
        """The same workload in blocks of S positions: the pool keeps at least its capacity in
        positions and holds the worst-case draw (every sequence at the longest length, the
        shared prefix and the copy-on-write targets)."""
        if self.prefix_len % S or (self.partition_size and self.partition_size % S):
            raise ValueError(f"block size {S} does not divide the prefix or the partitions")
        own = self.max_len - self.prefix_len
        need = self.num_seqs * -(-own // S) + self.prefix_len // S + self.cow_seqs
        scaled = -(-self.num_blocks * self.block_size // S)
        return self.replace(block_size=S, num_blocks=max(need, scaled),
                            description=f"{self.description}; block size {S}")


# The five serving-shaped workloads. Sizes: tiny fp32; 7B-like MHA; grouped-query;
# shared prefix with copy-on-write; long ragged context split into 512-token partitions.
CONFIGS = {
    "c1": Config("c1", 4, 4, 4, 64, 16, 32, "f32", 2470, "fixed", lens=(17, 33, 64, 5),
                 description="tiny fp32 paged decode, 4 seqs, 4/4 heads, D64, S16"),
    "c2": Config("c2", 64, 32, 32, 128, 16, 12000, "bf16", 2471, "uniform", len_lo=128,
                 len_hi=2048, description="MHA decode bf16, 64 seqs, 32/32 heads, D128, S16"),
    "c3": Config("c3", 128, 32, 8, 128, 16, 32768, "bf16", 2472, "uniform", len_lo=512,
                 len_hi=4096, description="GQA decode bf16, 128 seqs, 32/8 heads, D128, S16"),
    "c4": Config("c4", 256, 32, 8, 128, 16, 8320, "bf16", 2473, "prefix", len_lo=32,
                 len_hi=512, prefix_len=1024, cow_seqs=64,
                 description="prefix-shared decode bf16, 256 seqs, 1024-token shared prefix, "
                             "CoW x64, 32/8 heads, D128, S16"),
    "c5": Config("c5", 32, 64, 8, 128, 32, 32768, "bf16", 2474, "lognormal", len_lo=256,
                 len_hi=32768, lognormal_median=4096.0, lognormal_sigma=1.0,
                 partition_size=512,
                 description="long ragged split-context decode bf16, 32 seqs, 64/8 heads, "
                             "D128, S32, 512-token partitions"),
}

# Prefill workloads: a chunk of new tokens per sequence over its paged cache (chunked
# prefill), and whole prompts (the first forward pass of generation).
PREFILL = {
    "p1": Config("p1", 16, 32, 8, 128, 16, 8192, "bf16", 2475, "uniform", len_lo=1024,
                 len_hi=4096, query_len=512,
                 description="GQA chunked prefill bf16, 16 seqs, 512-token chunks over "
                             "contexts U[1024, 4096], 32/8 heads, D128, S16"),
    "p2": Config("p2", 8, 32, 8, 128, 16, 2048, "bf16", 2476, "uniform", len_lo=256,
                 len_hi=2048, query_len=-1,
                 description="GQA whole-prompt prefill bf16, 8 prompts U[256, 2048], "
                             "32/8 heads, D128, S16"),
}
PREFILL_SMALL = {
    "p1": PREFILL["p1"].replace(name="p1s", num_seqs=4, num_heads=8, num_kv_heads=2,
                                num_blocks=120, len_lo=40, len_hi=300, query_len=70),
    "p2": PREFILL["p2"].replace(name="p2s", num_seqs=3, num_heads=8, num_kv_heads=2,
                                num_blocks=60, len_lo=1, len_hi=200),
}

# Reduced versions with the same structure (ragged tails, several blocks and partitions,
# GQA groups, a shared prefix), small enough for the oracle to finish in well under a second.
SMALL = {
    "c1": CONFIGS["c1"],
    "c2": CONFIGS["c2"].replace(name="c2s", num_seqs=5, num_heads=4, num_kv_heads=4,
                                num_blocks=160, len_lo=1, len_hi=300),
    "c3": CONFIGS["c3"].replace(name="c3s", num_seqs=6, num_heads=8, num_kv_heads=2,
                                num_blocks=200, len_lo=1, len_hi=400),
    "c4": CONFIGS["c4"].replace(name="c4s", num_seqs=8, num_heads=8, num_kv_heads=2,
                                num_blocks=40, len_lo=1, len_hi=40, prefix_len=64,
                                cow_seqs=3),
    "c5": CONFIGS["c5"].replace(name="c5s", num_seqs=4, num_heads=16, num_kv_heads=2,
                                num_blocks=300, len_lo=1, len_hi=2000,
                                lognormal_median=300.0, partition_size=64),
}


class PoolExhausted(RuntimeError):
    """The physical pool has too few free blocks for the drawn lengths."""


@dataclass
class Workload:
    cfg: Config
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, MB]: the table decode reads (after any CoW redirect)
    block_tables_before: np.ndarray  # int32 [B, MB]: the table before copy-on-write
    block_mapping: np.ndarray  # int64 [M, 2]: (src, dst) copy-on-write pairs
    q: np.ndarray  # [B, H, D]
    k_cache: np.ndarray  # [N, Hkv, S, D]: pool before this step's copies and writes
    v_cache: np.ndarray  # [N, Hkv, (S / VS) D, VS], VS = min(S, 32)
    key: np.ndarray  # [B, Hkv, D]: newest token of each sequence
    value: np.ndarray  # [B, Hkv, D]
    slot_mapping: np.ndarray  # int64 [B]: slot = block_id * S + offset of that token
    logical_k: list | None = None  # per sequence [L_i, Hkv, D], the whole logical stream
    logical_v: list | None = None
    # Prefill workloads (query_len != 0): query tokens of sequence i are rows
    # query_start[i] .. query_start[i + 1] - 1 of q_prefill [T, H, D], at positions
    # L_i - Q_i .. L_i - 1; the pool then holds every position, the newest included.
    query_lens: np.ndarray | None = None  # int32 [B]
    query_start: np.ndarray | None = None  # int32 [B + 1]
    q_prefill: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def prefill_flops(self) -> int:
        """Multiply-adds x 2 of a prefill over the query tokens: each token at position p
        attends to p + 1 positions, for QK^T and for PV, in every q head."""
        c = self.cfg
        total = 0
        for L, Q in zip(self.context_lens.astype(np.int64), self.query_lens.astype(np.int64)):
            first = L - Q + 1  # positions attended by the first query token
            total += (first + L) * Q // 2
        return int(total) * c.num_heads * c.head_dim * 4

    def prefill_work_items(self, tile_tokens: int) -> np.ndarray:
        """Host-side prefill schedule: units i * T + t (sequence i, query tile t of tile_tokens
        tokens, T = tiles of the longest query) that have tokens, the most positions first."""
        Q = self.query_lens.astype(np.int64)
        L = self.context_lens.astype(np.int64)
        T = max(int(-(-Q.max() // tile_tokens)), 1) if len(Q) else 1
        units, cost = [], []
        for i in range(len(Q)):
            for t in range(-(-int(Q[i]) // tile_tokens)):
                last = min((t + 1) * tile_tokens, int(Q[i]))
                units.append(i * T + t)
                cost.append(int(L[i] - Q[i]) + last)
        order = np.argsort(-np.asarray(cost, dtype=np.int64), kind="stable")
        return np.asarray(units, dtype=np.int32)[order]

    def work_items(self, partition_size: int = 0) -> np.ndarray:
        """Host-side decode schedule: the units that have work, largest first.

        A unit is i * NP + p (sequence i, range p) with NP = 1 in single-pass mode (every
        sequence is listed, empty ones too: they get a zero row) and NP = ceil(max_context_len
        / partition_size) in split mode (only p < ceil(L_i / partition_size)). Ties keep index
        order. Any order gives the same result; largest-first lets small units fill in behind
        large ones."""
        L = self.context_lens.astype(np.int64)
        if partition_size <= 0:
            return np.argsort(-L, kind="stable").astype(np.int32)
        P = int(partition_size)
        NP = max(-(-self.max_context_len // P), 1)
        units, sizes = [], []
        for i, Li in enumerate(L):
            for p in range(-(-int(Li) // P)):
                units.append(i * NP + p)
                sizes.append(min(P, int(Li) - p * P))
        units = np.asarray(units, dtype=np.int64)
        order = np.argsort(-np.asarray(sizes, dtype=np.int64), kind="stable")
        return units[order].astype(np.int32)

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode call reads: sum_i L_i * Hkv * D * elt * 2."""
        c = self.cfg
        return self.total_tokens * c.num_kv_heads * c.head_dim * elt_bytes(c.dtype) * 2

    def unique_kv_bytes(self, include_copies: bool = True) -> int:
        """Distinct valid (block, kv head) rows touched by decode, K and V; by default plus the
        bytes the copy-on-write copies read (a step's unique reads), without them the decode
        launch's own unique reads."""
        c = self.cfg
        S = c.block_size
        seen = {}
        for i, L in enumerate(self.context_lens):
            nb = -(-int(L) // S)
            for j in range(nb):
                b = int(self.block_tables[i, j])
                rows = S if j < nb - 1 else int(L) - S * (nb - 1)
                seen[b] = max(seen.get(b, 0), rows)
        row_bytes = c.num_kv_heads * c.head_dim * elt_bytes(c.dtype) * 2
        copy_bytes = len(self.block_mapping) * S * row_bytes if include_copies else 0
        return sum(seen.values()) * row_bytes + copy_bytes


def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.len_dist == "fixed":
        L = np.array(cfg.lens, dtype=np.int64)
    elif cfg.len_dist == "uniform":
        L = rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.num_seqs, endpoint=True)
    elif cfg.len_dist == "lognormal":
        x = rng.lognormal(math.log(cfg.lognormal_median), cfg.lognormal_sigma, cfg.num_seqs)
        L = np.clip(np.rint(x), cfg.len_lo, cfg.len_hi).astype(np.int64)
    elif cfg.len_dist == "prefix":
        L = cfg.prefix_len + rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.num_seqs,
                                          endpoint=True)
    else:
        raise ValueError(f"unknown length distribution {cfg.len_dist!r}")
    assert len(L) == cfg.num_seqs
    return L.astype(np.int32)


def _fill(shape, dtype: str, poison: str, rng: np.random.Generator | None):
    st = storage_dtype(dtype)
    if poison == "nan":
        if dtype == "f32":
            return np.full(shape, _NAN_BITS["f32"], dtype=np.uint32).view(np.float32)
        return np.full(shape, _NAN_BITS[dtype], dtype=np.uint16).view(st)
    if poison == "zero":
        return np.zeros(shape, dtype=st)
    raise ValueError(f"unknown poison {poison!r}")


def generate(cfg: Config, poison: str = "nan", keep_logical: bool = False,
             lens: np.ndarray | None = None) -> Workload:
    """Build one workload.

    Draw order on one numpy Generator seeded with cfg.seed: lengths, one permutation of all
    pool ids (consumed in order as sequences need blocks), q, the logical K stream, the
    logical V stream; all values N(0,1) fp32, then rounded to the storage type (RNE).

    poison: what fills pool slots no sequence owns, including the tail of each sequence's
    last block and the newest token's slot: "nan" (correctness) or "zero" (timing).
    lens: optional override of the drawn lengths (edge-case tests); the draw still happens so
    that the rest of the stream is unchanged.
    """
    if cfg.dtype not in DTYPES:
        raise ValueError(cfg.dtype)
    if cfg.num_heads % cfg.num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    rng = np.random.default_rng(cfg.seed)
    L = draw_lengths(cfg, rng)
    if lens is not None:
        L = np.asarray(lens, dtype=np.int32)
        assert len(L) == cfg.num_seqs
    B, H, Hkv, D, S, N = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                          cfg.block_size, cfg.num_blocks)
    MB = max(cfg.max_blocks_per_seq, int(-(-int(L.max()) // S)) if B else 0, 1)
    perm = rng.permutation(N).astype(np.int32)
    cursor = 0

    def take(n):
        nonlocal cursor
        if cursor + n > N:
            raise PoolExhausted(f"{cfg.name}: need {cursor + n} blocks, pool has {N}")
        out = perm[cursor:cursor + n]
        cursor += n
        return out

    tables = np.full((B, MB), -1, dtype=np.int32)
    nblk = -(-L.astype(np.int64) // S)
    prefix = cfg.len_dist == "prefix"
    if prefix:
        if cfg.prefix_len % S:
            raise ValueError("prefix_len must be a multiple of block_size")
        npb = cfg.prefix_len // S
        shared = take(npb)
        for i in range(B):
            tables[i, :npb] = shared
            tables[i, npb:nblk[i]] = take(int(nblk[i]) - npb)
    else:
        for i in range(B):
            tables[i, :nblk[i]] = take(int(nblk[i]))

    # Copy-on-write of the last shared block for the first cow_seqs sequences.
    tables_before = tables.copy()
    mapping = np.zeros((0, 2), dtype=np.int64)
    if prefix and cfg.cow_seqs:
        fresh = take(cfg.cow_seqs)
        src = int(shared[-1])
        mapping = np.stack([np.full(cfg.cow_seqs, src), fresh]).T.astype(np.int64)
        tables[:cfg.cow_seqs, npb - 1] = fresh

    q = cast_from_f32(rng.standard_normal((B, H, D), dtype=np.float32), cfg.dtype)
    if prefix:
        n_stream = cfg.prefix_len + int((L - cfg.prefix_len).sum())
    else:
        n_stream = int(L.astype(np.int64).sum())
    ks = cast_from_f32(rng.standard_normal((n_stream, Hkv, D), dtype=np.float32), cfg.dtype)
    vs = cast_from_f32(rng.standard_normal((n_stream, Hkv, D), dtype=np.float32), cfg.dtype)

    # Row of the stream that holds logical position p of sequence i.
    seq_of, pos_of, row_of = [], [], []
    off = cfg.prefix_len if prefix else 0
    for i in range(B):
        Li = int(L[i])
        pos = np.arange(Li, dtype=np.int64)
        if prefix:
            rows = np.where(pos < cfg.prefix_len, pos, off + pos - cfg.prefix_len)
            off += Li - cfg.prefix_len
        else:
            rows = off + pos
            off += Li
        seq_of.append(np.full(Li, i, dtype=np.int64))
        pos_of.append(pos)
        row_of.append(rows)
    seq_of = np.concatenate(seq_of) if B else np.zeros(0, np.int64)
    pos_of = np.concatenate(pos_of) if B else np.zeros(0, np.int64)
    row_of = np.concatenate(row_of) if B else np.zeros(0, np.int64)

    # The pool before a decode step holds every position except each sequence's newest one
    # (a prefill reads them all). Shared prefix positions are placed through sequence 0's
    # (pre-CoW) table only.
    newest = pos_of == (L[seq_of].astype(np.int64) - 1)
    place = ~newest if cfg.query_len == 0 else np.ones_like(newest)
    if prefix:
        place &= (pos_of >= cfg.prefix_len) | (seq_of == 0)
    blk = tables_before[seq_of[place], pos_of[place] // S].astype(np.int64)
    slot_off = pos_of[place] % S
    VS = v_group(S)
    k_cache = _fill((N, Hkv, S, D), cfg.dtype, poison, rng)
    v_cache = _fill((N, Hkv, (S // VS) * D, VS), cfg.dtype, poison, rng)
    k_cache[blk, :, slot_off, :] = ks[row_of[place]]
    v_cache.reshape(N, Hkv, S // VS, D, VS)[blk, :, slot_off // VS, :, slot_off % VS] = \
        vs[row_of[place]]

    # Newest token of each sequence: written by reshape_and_cache during the step. A sequence
    # with an empty context has none: its slot is -1 (skipped) and its rows are zero.
    has = L > 0
    key = np.zeros((B, Hkv, D), dtype=ks.dtype)
    value = np.zeros((B, Hkv, D), dtype=vs.dtype)
    key[has] = ks[row_of[newest]]
    value[has] = vs[row_of[newest]]
    lp = np.maximum(L.astype(np.int64) - 1, 0)
    slot_mapping = np.where(has, tables[np.arange(B), lp // S].astype(np.int64) * S + lp % S, -1)
    if prefix and np.any(L.astype(np.int64) - 1 < cfg.prefix_len):
        raise ValueError("prefix configs need a non-empty suffix")

    wl = Workload(cfg=cfg, context_lens=L, block_tables=tables,
                  block_tables_before=tables_before, block_mapping=mapping, q=q,
                  k_cache=k_cache, v_cache=v_cache, key=key, value=value,
                  slot_mapping=slot_mapping.astype(np.int64))
    wl.meta["blocks_used"] = cursor
    if cfg.query_len != 0:
        Qn = L.astype(np.int64) if cfg.query_len < 0 else np.minimum(L, cfg.query_len)
        wl.query_lens = Qn.astype(np.int32)
        wl.query_start = np.concatenate([[0], np.cumsum(Qn)]).astype(np.int32)
        wl.q_prefill = cast_from_f32(
            rng.standard_normal((int(Qn.sum()), H, D), dtype=np.float32), cfg.dtype)
    if keep_logical:
        starts = np.concatenate([[0], np.cumsum(L.astype(np.int64))])
        wl.logical_k = [ks[row_of[starts[i]:starts[i + 1]]] for i in range(B)]
        wl.logical_v = [vs[row_of[starts[i]:starts[i + 1]]] for i in range(B)]
    return wl


def permute_pool(wl: Workload, seed: int) -> Workload:
    """The same workload with its physical blocks relabelled by a seeded permutation.

    Tables, slots and CoW pairs are rewritten to follow the blocks, so what every sequence
    attends over is unchanged; only where the bytes live moves."""
    cfg = wl.cfg
    N, S = cfg.num_blocks, cfg.block_size
    pi = np.random.default_rng(seed).permutation(N)  # old id b moves to pi[b]
    k = np.empty_like(wl.k_cache)
    v = np.empty_like(wl.v_cache)
    k[pi] = wl.k_cache
    v[pi] = wl.v_cache

    def remap(t):
        t = t.copy()
        m = t >= 0
        t[m] = pi[t[m]]
        return t

    slots = wl.slot_mapping
    new_slots = np.where(slots >= 0, pi[slots // S] * S + slots % S, slots)
    return dataclasses.replace(
        wl, k_cache=k, v_cache=v, block_tables=remap(wl.block_tables),
        block_tables_before=remap(wl.block_tables_before),
        block_mapping=pi[wl.block_mapping].astype(np.int64) if len(wl.block_mapping)
        else wl.block_mapping, slot_mapping=new_slots.astype(np.int64), meta=dict(wl.meta))


def contiguous_layout(wl: Workload) -> Workload:
    """The same workload in the conventional contiguous reservation: sequence i owns pool
    blocks i * MB .. i * MB + MB - 1 in order (the per-request maximum-length reservation that
    paging replaces). Tables are rewritten to that identity mapping, so decode can run either
    through them or table-free; prefix sharing and copy-on-write do not exist in this layout."""
    cfg = wl.cfg
    if len(wl.block_mapping):
        raise ValueError("a contiguous reservation has no shared blocks")
    B, MB, S = cfg.num_seqs, wl.block_tables.shape[1], cfg.block_size
    N = B * MB
    k = np.zeros((N,) + wl.k_cache.shape[1:], dtype=wl.k_cache.dtype)
    v = np.zeros((N,) + wl.v_cache.shape[1:], dtype=wl.v_cache.dtype)
    tables = np.full_like(wl.block_tables, -1)
    for i in range(B):
        nb = -(-int(wl.context_lens[i]) // S)
        old = wl.block_tables[i, :nb]
        k[i * MB:i * MB + nb] = wl.k_cache[old]
        v[i * MB:i * MB + nb] = wl.v_cache[old]
        tables[i, :nb] = i * MB + np.arange(nb)
    slots = wl.slot_mapping.copy()
    for i, s_ in enumerate(slots):
        if s_ >= 0:
            j = int(wl.context_lens[i] - 1) // S
            slots[i] = (i * MB + j) * S + s_ % S
    return dataclasses.replace(wl, cfg=cfg.replace(num_blocks=N), k_cache=k, v_cache=v,
                               block_tables=tables, block_tables_before=tables.copy(),
                               slot_mapping=slots, meta=dict(wl.meta))
