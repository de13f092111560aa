"""Host planning of a decode step over shared prefix blocks (CPU): the groups share their
tables over the shared partition, and the grouped partition 0 plus the work list cover every
unit with positions exactly once."""
from __future__ import annotations

import numpy as np
import pytest

from paged_kv_cache_247_amd import contract as C
from paged_kv_cache_247_amd import sharing
from paged_kv_cache_247_amd import workload as W


def _units(wl, P):
    NP = -(-wl.max_context_len // P)
    return {i * NP + p for i, L in enumerate(wl.context_lens.tolist())
            for p in range(NP) if p * P < L}


@pytest.mark.parametrize("heads,width", [(8, 4), (16, 2), (4, 4)])
def test_plan_on_the_prefix_workload(heads, width):
    cfg = W.SMALL["c4"].replace(num_heads=heads)
    wl = W.generate(cfg)
    S = cfg.block_size
    assert sharing.group_width(cfg.group) == width
    plan = sharing.plan(wl.block_tables, wl.context_lens, S, wl.max_context_len, cfg.group)
    # copy-on-write gives some sequences a private last prefix block: the shared part is
    # the blocks before it
    assert plan.partition_size == (cfg.prefix_len // S - 1) * S
    g = plan.groups
    assert g.shape[1] == 4 and ((g >= 0).sum(axis=1) <= width).all()
    C.check_groups(g, wl.block_tables, wl.context_lens, plan.partition_size, S,
                   cfg.num_blocks, cfg.group)
    members = g[g >= 0]
    assert len(members) == len(set(members.tolist())) == cfg.num_seqs
    covered = {int(m) * plan.num_partitions for m in members}
    items = set(plan.work_items.tolist())
    assert len(items) == len(plan.work_items) and not covered & items
    assert covered | items == _units(wl, plan.partition_size)
    sizes = [min(plan.partition_size,
                 int(wl.context_lens[u // plan.num_partitions])
                 - (u % plan.num_partitions) * plan.partition_size) for u in plan.work_items]
    assert sizes == sorted(sizes, reverse=True)


def test_no_plan_without_shared_blocks():
    wl = W.generate(W.SMALL["c3"])
    assert sharing.plan(wl.block_tables, wl.context_lens, 16, wl.max_context_len, 4) is None
    assert sharing.group_width(16) == 1 and sharing.group_width(1) == 4


def test_common_prefix_blocks():
    t = np.array([[5, 6, 7, 8], [5, 6, 9, 1], [5, 6, 7, 2]], np.int32)
    assert sharing.common_prefix_blocks(t, np.array([64, 64, 64]), 16) == 2
    assert sharing.common_prefix_blocks(t, np.array([20, 64, 64]), 16) == 1  # one full block
    assert sharing.common_prefix_blocks(t[[0, 2]], np.array([48, 64]), 16) == 3


def test_group_contract_violations():
    wl = W.generate(W.SMALL["c4"])
    S, N = 16, wl.cfg.num_blocks
    plan = sharing.plan(wl.block_tables, wl.context_lens, S, wl.max_context_len, 4)
    P = plan.partition_size
    ok = plan.groups

    def bad(groups=ok, tables=wl.block_tables, lens=wl.context_lens):
        with pytest.raises(C.ContractError):
            C.check_groups(groups, tables, lens, P, S, N, 4)

    g = ok.copy(); g[1, 0] = g[0, 1]
    bad(groups=g)                                    # a sequence in two groups
    g = ok.copy(); g[0, 0] = -1
    bad(groups=g)                                    # no first member
    with pytest.raises(C.ContractError):             # more members than 16 / G columns hold
        C.check_groups(ok, wl.block_tables, wl.context_lens, P, S, N, 8)
    t = wl.block_tables.copy(); t[ok[0, 1], 0] = t[ok[0, 1], 0] + 1
    bad(tables=t)                                    # a member's table differs
    L = wl.context_lens.copy(); L[ok[0, 2]] = P - 1
    bad(lens=L)                                      # too short for the shared partition


def test_group_contract_with_the_work_list():
    """Groups run in one launch with the step's work list: the list must not name a member's
    partition 0, and with the fused newest-position write each member reaches past the shared
    partition."""
    wl = W.generate(W.SMALL["c4"])
    S, N = 16, wl.cfg.num_blocks
    plan = sharing.plan(wl.block_tables, wl.context_lens, S, wl.max_context_len, 4)
    P, NP, g = plan.partition_size, plan.num_partitions, plan.groups
    C.check_groups(g, wl.block_tables, wl.context_lens, P, S, N, 4,
                   work_items=plan.work_items, num_partitions=NP, fused_write=True)
    with pytest.raises(C.ContractError, match="partition 0"):
        C.check_groups(g, wl.block_tables, wl.context_lens, P, S, N, 4,
                       work_items=np.append(plan.work_items, g[1, 1] * NP), num_partitions=NP)
    L = wl.context_lens.copy(); L[g[0, 1]] = P
    C.check_groups(g, wl.block_tables, L, P, S, N, 4)  # reaches the partition's end
    with pytest.raises(C.ContractError):             # but the newest position would be in it
        C.check_groups(g, wl.block_tables, L, P, S, N, 4, work_items=plan.work_items,
                       num_partitions=NP, fused_write=True)


@pytest.mark.parametrize("heads,width", [(8, 4), (16, 2), (4, 4), (32, 1)])
def test_whole_plan_covers_every_sequence_once(heads, width):
    cfg = W.SMALL["c4"].replace(num_heads=heads)
    wl = W.generate(cfg)
    S = cfg.block_size
    plan = sharing.plan_whole(wl.block_tables, wl.context_lens, S, cfg.group)
    if width == 1:  # one sequence per group: grouping would save no read
        assert plan is None
        plan = sharing.plan_whole(wl.block_tables, wl.context_lens, S, cfg.group,
                                  prefix_blocks=cfg.prefix_len // S - 1)
    assert plan is not None and plan.shared_len == (cfg.prefix_len // S - 1) * S
    g = plan.groups
    assert g.shape[1] == 4 and ((g >= 0).sum(axis=1) <= width).all() and (g[:, 0] >= 0).all()
    members = g[g >= 0]
    assert sorted(members.tolist()) == list(range(cfg.num_seqs))
    C.check_whole_groups(g, wl.block_tables, wl.context_lens, plan.shared_len, S,
                         cfg.num_blocks, cfg.group, fused_write=True)
    load = [plan.shared_len + sum(int(wl.context_lens[m]) - plan.shared_len for m in row if m >= 0)
            for row in g]
    assert load == sorted(load, reverse=True)


def test_whole_plan_balances_the_groups():
    """The prefix-shared batch: 256 sequences in 64 groups of four whose own positions (past
    the shared 1008) differ by little; every group holds four members."""
    cfg = W.CONFIGS["c4"]
    wl = W.generate(cfg, poison="zero")
    plan = sharing.plan_whole(wl.block_tables, wl.context_lens, cfg.block_size, cfg.group)
    assert plan.shared_len == 1008 and plan.groups.shape == (64, 4) and (plan.groups >= 0).all()
    own = [sum(int(wl.context_lens[m]) - plan.shared_len for m in row) for row in plan.groups]
    assert max(own) - min(own) <= 0.05 * np.mean(own)


def test_whole_plan_needs_every_sequence_past_the_shared_part():
    wl = W.generate(W.SMALL["c4"])
    L = wl.context_lens.copy()
    plan = sharing.plan_whole(wl.block_tables, L, 16, 4)
    L[2] = plan.shared_len  # the newest position would fall in the shared part
    assert sharing.plan_whole(wl.block_tables, L, 16, 4, prefix_blocks=plan.shared_len // 16) is None
    assert sharing.plan_whole(wl.block_tables, L, 16, 4, newest_outside=False,
                              prefix_blocks=plan.shared_len // 16) is not None
    assert sharing.plan_whole(W.generate(W.SMALL["c3"]).block_tables,
                              W.generate(W.SMALL["c3"]).context_lens, 16, 4) is None


def test_whole_group_contract_violations():
    wl = W.generate(W.SMALL["c4"])
    c = wl.cfg
    plan = sharing.plan_whole(wl.block_tables, wl.context_lens, c.block_size, c.group)
    args = (wl.block_tables, wl.context_lens, plan.shared_len, c.block_size, c.num_blocks, c.group)
    C.check_whole_groups(plan.groups, *args, fused_write=True)
    bad = plan.groups.copy()
    bad[0, 1] = bad[1, 0]  # a sequence in two groups
    with pytest.raises(C.ContractError):
        C.check_whole_groups(bad, *args)
    tables = wl.block_tables.copy()
    m = int(plan.groups[0, 1])
    tables[m, 0] = (tables[m, 0] + 1) % c.num_blocks  # a member disagrees over the shared part
    with pytest.raises(C.ContractError):
        C.check_whole_groups(plan.groups, tables, *args[1:])
    tables = wl.block_tables.copy()
    nb = -(-int(wl.context_lens[m]) // c.block_size)
    tables[m, nb - 1] = c.num_blocks  # a member's own block outside the pool
    with pytest.raises(C.ContractError):
        C.check_whole_groups(plan.groups, tables, *args[1:])
