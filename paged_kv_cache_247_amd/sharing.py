"""Host planning of a decode step over shared prefix blocks.

Requests that share a prompt prefix share its KV blocks (Hacker News discussion of
PagedAttention, replies on prefix sharing), so their block tables agree over the prefix. A
decode step can then read each shared tile once for several sequences
(pkv_paged_attention_decode_shared, up to 16 / G sequences per group) instead of once per
sequence. The step works on split-context partitions of P positions, with P a multiple of the
block size inside the shared prefix, in two launches:

  1. partition 0 of every grouped sequence, one pass per group, and in the same launch every
     other unit (i, p) with positions -- p >= 1 of grouped sequences, all partitions of the
     others -- as split-context decode runs them, from a work list ordered largest first;
  2. the merge of the partitions (pkv_paged_attention_reduce).

The result is the same attention (the merge is an exact rewriting of the softmax sum); only
the order of the fp32 additions differs from a single pass.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def common_prefix_blocks(block_tables: np.ndarray, context_lens: np.ndarray,
                         block_size: int) -> int:
    """Leading table entries that every sequence with a non-empty context holds in common
    (entries wholly inside its context only)."""
    L = np.asarray(context_lens).astype(np.int64)
    rows = np.asarray(block_tables)[L > 0]
    if not len(rows):
        return 0
    full = int((L[L > 0] // block_size).min())  # entries every sequence fills completely
    same = np.all(rows[:, :full] == rows[:1, :full], axis=0)
    return int(full if same.all() else np.argmin(same))


def _classes(tables: np.ndarray, L: np.ndarray, nb: int, need: int) -> list[list[int]]:
    """Sequences with at least `need` positions, grouped by their first nb table entries."""
    classes: dict[bytes, list[int]] = {}
    for i in np.flatnonzero(L >= need).tolist():
        classes.setdefault(tables[i, :nb].tobytes(), []).append(i)
    return [m for m in classes.values() if len(m) >= 2]


def best_prefix_blocks(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                       width: int, newest_outside: bool = True) -> int:
    """The shared partition length (in blocks) that saves the most tile reads: for nb blocks,
    each class of sequences agreeing over nb entries reads them once per group of `width`
    instead of once per sequence. 0 if no two sequences share a block."""
    S = int(block_size)
    L = np.asarray(context_lens).astype(np.int64)
    tables = np.asarray(block_tables)
    top = int((L // S).max()) if len(L) else 0
    best, gain = 0, 0
    for nb in range(1, top + 1):
        g = sum((len(m) - -(-len(m) // width)) * nb
                for m in _classes(tables, L, nb, nb * S + (1 if newest_outside else 0)))
        if g > gain:
            best, gain = nb, g
    return best


@dataclasses.dataclass
class SharedPlan:
    partition_size: int       # P
    num_partitions: int       # NP = ceil(max_context_len / P)
    groups: np.ndarray        # int32 [num_groups, 4], -1 pads
    work_items: np.ndarray    # int32 units i * NP + p for launch 2, largest first


def group_width(group: int) -> int:
    """Sequences per group for a query group of G heads: the 16 product columns hold G heads
    of each member (at most 4 members, the width of a group row)."""
    return max(1, min(4, 16 // max(int(group), 1)))


def plan(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
         max_context_len: int, group: int, max_members: int | None = None,
         prefix_blocks: int | None = None, newest_outside: bool = True) -> SharedPlan | None:
    """Groups of up to group_width(group) sequences (fewer if max_members says so), G = group
    query heads per kv head, whose tables agree over the first prefix_blocks entries (default:
    the length that saves the most tile reads, see best_prefix_blocks).
    A sequence joins a group only if its context reaches past the prefix (past it by one more
    position when the step also writes the newest token: that token must not fall in the
    shared partition). None if no two sequences can share."""
    S = int(block_size)
    L = np.asarray(context_lens).astype(np.int64)
    tables = np.asarray(block_tables)
    width = group_width(group)
    if max_members is not None:
        width = max(1, min(width, int(max_members)))
    nb = (best_prefix_blocks(tables, L, S, width, newest_outside) if prefix_blocks is None
          else int(prefix_blocks))
    if nb <= 0:
        return None
    P = nb * S
    groups = []
    for members in _classes(tables, L, nb, P + (1 if newest_outside else 0)):
        for k in range(0, len(members), width):
            chunk = members[k:k + width]
            groups.append(chunk + [-1] * (4 - len(chunk)))
    if not groups:
        return None
    groups = np.asarray(groups, dtype=np.int32).reshape(-1, 4)
    NP = -(-int(max_context_len) // P)
    grouped = np.zeros(len(L), dtype=bool)
    grouped[groups[groups >= 0]] = True
    units, sizes = [], []
    for i in range(len(L)):
        for p in range(1 if grouped[i] else 0, NP):
            n = min(P, int(L[i]) - p * P)
            if n > 0:  # an empty context needs no unit: the merge writes zeros for it
                units.append(i * NP + p)
                sizes.append(n)
    order = np.argsort(-np.asarray(sizes, dtype=np.int64), kind="stable")
    items = np.asarray(units, dtype=np.int32)[order] if units else np.zeros(0, np.int32)
    return SharedPlan(P, NP, groups, items)


@dataclasses.dataclass
class WholePlan:
    shared_len: int           # positions every member of a group shares (a multiple of S)
    groups: np.ndarray        # int32 [num_groups, 4], -1 pads, most positions first


def plan_whole(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
               group: int, newest_outside: bool = True,
               prefix_blocks: int | None = None) -> WholePlan | None:
    """Groups for pkv_paged_attention_decode_grouped: every sequence in exactly one group of up
    to group_width(group) sequences whose tables agree over the first prefix_blocks entries
    (default: the length that saves the most tile reads, see best_prefix_blocks); a sequence
    sharing with none is a group of its own. Within a class of sequences that agree, members are
    dealt to the class's groups longest own part first onto the group with the fewest own
    positions, so the groups' work is even; groups are listed with the most positions first.
    None when some sequence is too short for the shared length (it must reach past it, by one
    more position when the step writes the newest token) or nothing is shared."""
    S = int(block_size)
    L = np.asarray(context_lens).astype(np.int64)
    tables = np.asarray(block_tables)
    width = group_width(group)
    nb = (best_prefix_blocks(tables, L, S, width, newest_outside) if prefix_blocks is None
          else int(prefix_blocks))
    if nb <= 0 or not len(L):
        return None
    P = nb * S
    need = P + (1 if newest_outside else 0)
    if (L < need).any():
        return None
    classes: dict[bytes, list[int]] = {}
    for i in range(len(L)):
        classes.setdefault(tables[i, :nb].tobytes(), []).append(i)
    groups, loads = [], []
    for members in classes.values():
        ng = -(-len(members) // width)
        rows = [[] for _ in range(ng)]
        load = [0] * ng
        for i in sorted(members, key=lambda m: -int(L[m])):
            k = min((j for j in range(ng) if len(rows[j]) < width), key=lambda j: load[j])
            rows[k].append(i)
            load[k] += int(L[i]) - P
        for row, ld in zip(rows, load):
            groups.append(row + [-1] * (4 - len(row)))
            loads.append(P + ld)
    order = np.argsort(-np.asarray(loads, dtype=np.int64), kind="stable")
    return WholePlan(P, np.asarray(groups, dtype=np.int32).reshape(-1, 4)[order])
