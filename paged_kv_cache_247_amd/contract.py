"""Host-side checks of the caller contract of the C ABI (include/pagedkv.h).

The library validates shapes, sizes and pointers itself, but not the contents of device
buffers -- block ids, lengths, slots, copy pairs -- since that would cost a device-to-host copy
on every call. With PKV_VALIDATE=1 in the environment the Python binding copies those buffers
to the host and runs these checks before anything is enqueued; a violation raises
PagedKVError (invalid argument). Each function takes numpy arrays and raises ContractError
(a ValueError) naming the first violation.

What is checked (the contract the kernels rely on; a violation never makes a kernel touch
memory outside its buffers, since they clamp ids and lengths, but the affected results are
undefined):
  * decode: 0 <= L_i <= max_context_len <= MB * S; every table entry a sequence uses
    (j < ceil(L_i / S)) names a pool block; with the fused newest-token write, no two
    sequences write the same slot; a work list names units in range, each at most once.
  * cache write: non-negative slots are distinct and inside the pool (N * S slots).
  * block copies: sources and destinations inside the pool, destinations distinct, no
    destination also a source, no pair copying a block onto itself.
  * prefill: query_start runs from 0 to T without decreasing, Q_i <= max_query_len,
    Q_i <= L_i <= MB * S, and the used table entries name pool blocks.
"""
from __future__ import annotations

import numpy as np


class ContractError(ValueError):
    """A device buffer's contents break the caller contract."""


def _fail(msg: str):
    raise ContractError(msg)


def _check_lengths(L: np.ndarray, bound: int, MB: int, S: int):
    if len(L) and L.min() < 0:
        _fail(f"context_lens[{int(np.argmin(L))}] = {int(L.min())} is negative")
    if bound > MB * S:
        _fail(f"max_context_len {bound} exceeds max_blocks_per_seq * block_size = {MB * S}")
    if len(L) and L.max() > bound:
        i = int(np.argmax(L))
        _fail(f"context_lens[{i}] = {int(L[i])} exceeds the bound {bound}")


def _check_tables(tables: np.ndarray, L: np.ndarray, S: int, num_blocks: int):
    used = -(-L.astype(np.int64) // S)
    cols = np.arange(tables.shape[1])[None, :]
    mask = cols < used[:, None]
    bad = mask & ((tables < 0) | (tables >= num_blocks))
    if bad.any():
        i, j = map(int, np.argwhere(bad)[0])
        _fail(f"block_tables[{i}, {j}] = {int(tables[i, j])} is not a pool block "
              f"(pool of {num_blocks}; sequence {i} uses {int(used[i])} entries)")


def check_decode(block_tables, context_lens, max_context_len: int, block_size: int,
                 num_blocks: int, max_blocks_per_seq: int, partition_size: int = 0,
                 work_items=None, fused_write: bool = False):
    """block_tables [B, MB] int32 (None: the contiguous reservation), context_lens [B],
    work_items: optional unit list (units i * NP + p)."""
    L = np.asarray(context_lens).astype(np.int64)
    S, MB = int(block_size), int(max_blocks_per_seq)
    _check_lengths(L, int(max_context_len), MB, S)
    B = len(L)
    if block_tables is None:
        tables = np.arange(B, dtype=np.int64)[:, None] * MB + np.arange(MB)[None, :]
    else:
        tables = np.asarray(block_tables).astype(np.int64)
    _check_tables(tables, L, S, num_blocks)
    if fused_write:
        live = np.flatnonzero(L > 0)
        p = L[live] - 1
        slots = tables[live, p // S] * S + p % S
        u, counts = np.unique(slots, return_counts=True)
        if (counts > 1).any():
            s = int(u[np.argmax(counts)])
            who = live[slots == s].tolist()
            _fail(f"sequences {who} would write their newest token to the same slot {s}")
    if work_items is not None:
        w = np.asarray(work_items).astype(np.int64)
        P = int(partition_size)
        NP = -(-int(max_context_len) // P) if P > 0 else 1
        if len(w) and (w.min() < 0 or w.max() >= B * max(NP, 1)):
            _fail(f"work item outside [0, {B * max(NP, 1)}): {int(w.min())}..{int(w.max())}")
        u, counts = np.unique(w, return_counts=True)
        if (counts > 1).any():
            _fail(f"work item {int(u[np.argmax(counts)])} listed more than once")


def check_slots(slot_mapping, block_size: int, num_blocks: int):
    """Non-negative slots distinct and inside the pool (negative slots are skipped)."""
    s = np.asarray(slot_mapping).astype(np.int64)
    live = s[s >= 0]
    if len(live) and live.max() >= num_blocks * block_size:
        _fail(f"slot {int(live.max())} is outside the pool of {num_blocks * block_size} slots")
    u, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        _fail(f"slot {int(u[np.argmax(counts)])} is written by more than one token")


def check_copy_pairs(block_mapping, num_blocks: int):
    """[M, 2] (src, dst) pairs."""
    m = np.asarray(block_mapping).astype(np.int64).reshape(-1, 2)
    if not len(m):
        return
    src, dst = m[:, 0], m[:, 1]
    if min(src.min(), dst.min()) < 0 or max(src.max(), dst.max()) >= num_blocks:
        _fail(f"a copy pair names a block outside the pool of {num_blocks}")
    if (src == dst).any():
        _fail(f"pair {int(np.argmax(src == dst))} copies block {int(src[src == dst][0])} "
              "onto itself")
    u, counts = np.unique(dst, return_counts=True)
    if (counts > 1).any():
        _fail(f"block {int(u[np.argmax(counts)])} is the destination of more than one pair")
    both = np.intersect1d(src, dst)
    if len(both):
        _fail(f"block {int(both[0])} is both a source and a destination")


def check_groups(groups, block_tables, context_lens, partition_size: int, block_size: int,
                 num_blocks: int, group: int, work_items=None, num_partitions: int = 1,
                 fused_write: bool = False):
    """Groups for the shared-prefix decode: [n, 4] sequence ids, -1 pads; the first entry of a
    row is a sequence; a sequence in at most one group; every member's context covers the
    shared partition (reaches past it with the fused newest-position write) and its table
    agrees with the first member's over it; a work list run in the same launch (units
    i * num_partitions + p) holds no member's partition 0."""
    gm = np.asarray(groups).astype(np.int64).reshape(-1, 4)
    L = np.asarray(context_lens).astype(np.int64)
    tables = np.asarray(block_tables).astype(np.int64)
    B, P, S = len(L), int(partition_size), int(block_size)
    width = max(1, min(4, 16 // max(int(group), 1)))
    used = gm[:, :width]
    if len(gm) and (gm[:, 0] < 0).any():
        _fail(f"group {int(np.argmax(gm[:, 0] < 0))} has no first member")
    if (gm[:, width:] != -1).any():
        _fail(f"a group lists more than {width} sequences (16 columns over {group} heads)")
    if ((used < -1) | (used >= B)).any():
        _fail("a group names a sequence outside the batch")
    live = used[used >= 0]
    u, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        _fail(f"sequence {int(u[np.argmax(counts)])} is in more than one group")
    nb = P // S
    need = P + (1 if fused_write else 0)
    for k, row in enumerate(used.tolist()):
        members = [m for m in row if m >= 0]
        for m in members:
            if L[m] < need:
                _fail(f"group {k}: sequence {m} has {int(L[m])} positions, the shared "
                      f"partition needs {need}")
            if not np.array_equal(tables[m, :nb], tables[members[0], :nb]):
                _fail(f"group {k}: sequence {m}'s table differs from sequence {members[0]}'s "
                      f"within the shared partition")
        ids = tables[members[0], :nb]
        if len(ids) and (ids.min() < 0 or ids.max() >= num_blocks):
            _fail(f"group {k}: a shared table entry is not a pool block")
    if work_items is not None and len(live):
        first = np.asarray(work_items).astype(np.int64)
        both = np.intersect1d(first, live * max(int(num_partitions), 1))
        if len(both):
            _fail(f"work item {int(both[0])} is partition 0 of a grouped sequence")


def check_whole_groups(groups, block_tables, context_lens, shared_len: int, block_size: int,
                       num_blocks: int, group: int, fused_write: bool = False):
    """Groups for the whole-group decode: as check_groups over the shared positions, and every
    table entry a member uses (its first ceil(L / S)) names a pool block."""
    check_groups(groups, block_tables, context_lens, shared_len, block_size, num_blocks, group,
                 fused_write=fused_write)
    gm = np.asarray(groups).astype(np.int64).reshape(-1, 4)
    L = np.asarray(context_lens).astype(np.int64)
    tables = np.asarray(block_tables).astype(np.int64)
    S = int(block_size)
    for m in gm[gm >= 0].tolist():
        nb = -(-int(L[m]) // S)
        if nb > tables.shape[1]:
            _fail(f"sequence {m} has {int(L[m])} positions, its table row holds {tables.shape[1]} blocks")
        ids = tables[m, :nb]
        if len(ids) and (ids.min() < 0 or ids.max() >= num_blocks):
            _fail(f"sequence {m}: a used table entry is not a pool block")


def check_prefill(block_tables, context_lens, query_start, max_query_len: int, block_size: int,
                  num_blocks: int, num_tokens: int):
    L = np.asarray(context_lens).astype(np.int64)
    qs = np.asarray(query_start).astype(np.int64)
    tables = np.asarray(block_tables).astype(np.int64)
    S, MB = int(block_size), tables.shape[1]
    if len(qs) != len(L) + 1 or qs[0] != 0 or qs[-1] != num_tokens:
        _fail(f"query_start must run from 0 to num_tokens = {num_tokens}")
    Q = np.diff(qs)
    if (Q < 0).any():
        _fail(f"query_start decreases at sequence {int(np.argmax(Q < 0))}")
    if len(Q) and Q.max() > max_query_len:
        _fail(f"sequence {int(np.argmax(Q))} has {int(Q.max())} query tokens, over "
              f"max_query_len {max_query_len}")
    if (Q > L).any():
        i = int(np.argmax(Q > L))
        _fail(f"sequence {i} has {int(Q[i])} query tokens but a context of {int(L[i])}")
    _check_lengths(L, MB * S, MB, S)
    _check_tables(tables, L, S, num_blocks)
