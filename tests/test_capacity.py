"""The capacity and waste model of contiguous reservation vs paged allocation, pinned to the
worked example and sizing formula of Qualiteg's "About PagedAttention for LLM serving" and to
closed forms."""
from __future__ import annotations

import numpy as np
import pytest

from paged_kv_cache_247_amd import capacity as C
from paged_kv_cache_247_amd import workload as W


def test_worked_example_of_the_post():
    # "Deepening Our Understanding ...": 1024 positions reserved, 13 generated, 1011 wasted.
    reserved, used = 1024, 13
    assert reserved - used == 1011
    assert C.waste_fraction(used, reserved) == pytest.approx(1011 / 1024)
    # the same request under paging with 16-position blocks holds one block: 3 wasted
    held = int(C.paged_positions(np.array([used]), 16)[0])
    assert held == 16 and held - used == 3


def test_sizing_formula_solved_for_users():
    # total = weights + users * max_context * kv_per_token, solved for users (floor)
    bpt = C.kv_bytes_per_token(32, 8, 128, 2)
    assert bpt == 2 * 32 * 8 * 128 * 2 == 131072
    gib = 2 ** 30
    assert C.contiguous_users(288 * gib, 16 * gib, 4096, bpt) == (272 * gib) // (4096 * bpt) == 544
    assert C.contiguous_users(10 * gib, 16 * gib, 4096, bpt) == 0
    users = C.contiguous_users(100 * gib, 4 * gib, 1000, 12345)
    assert 4 * gib + users * 1000 * 12345 <= 100 * gib < 4 * gib + (users + 1) * 1000 * 12345


@pytest.mark.parametrize("S", [1, 16, 32, 256])
def test_paged_waste_is_below_one_block(S):
    L = np.arange(1, 5000)
    held = C.paged_positions(L, S)
    assert np.all(held >= L) and np.all(held - L <= S - 1)
    assert np.all(held % S == 0)
    assert np.all(held[L % S == 0] == L[L % S == 0])


@pytest.mark.parametrize("S", [16, 64, 256])
def test_mean_waste_over_full_residue_cycles(S):
    # lengths covering every residue mod S equally often waste (S - 1) / 2 positions on average
    L = np.arange(1, 20 * S + 1)
    assert float((C.paged_positions(L, S) - L).mean()) == (S - 1) / 2


def test_shared_prefix_holds_the_prefix_once():
    lens = np.array([1030, 1040, 1024 + 33])
    # 64 shared blocks, then ceil(6/16) + ceil(16/16) + ceil(33/16) = 1 + 1 + 3 own blocks
    assert C.shared_prefix_positions(lens, 1024, 16) == 1024 + 5 * 16
    # a prefix that ends mid-block: only whole blocks are shared
    assert C.shared_prefix_positions(np.array([40, 40]), 20, 16) == 16 + 2 * 32


def test_paged_admission_in_arrival_order():
    lens = np.array([10, 20, 30, 40])  # S = 16 holds 16, 32, 32, 48
    assert C.paged_users(lens, 16, 16) == 1
    assert C.paged_users(lens, 79, 16) == 2
    assert C.paged_users(lens, 80, 16) == 3
    assert C.paged_users(lens, 10**6, 16) == 4
    assert C.paged_users(lens, 15, 16) == 0


def test_model_rows_on_the_workload_distributions():
    rows = C.model(names=("c3", "c5"), block_sizes=(16, 256), sample=20_000)
    by = {(r.workload, r.block_size): r for r in rows}
    for name in ("c3", "c5"):
        cfg = W.CONFIGS[name]
        small, big = by[(name, 16)], by[(name, 256)]
        # larger blocks waste more (the post's fragmentation remark) but stay far below the
        # contiguous reservation's waste
        assert small.paged_waste < big.paged_waste < small.contiguous_waste
        assert small.paged_users >= big.paged_users > small.contiguous_users
        assert small.max_context == cfg.max_len
    # uniform [512, 4096]: contiguous waste = 1 - E[L] / 4096 = 1 - 2304 / 4096
    assert by[("c3", 16)].contiguous_waste == pytest.approx(1 - 2304 / 4096, abs=0.01)
