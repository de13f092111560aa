"""Pins of the prefill oracle (CPU): torch's scaled-dot-product attention on the logical
stream with the causal mask of each chunk, the decode oracle for one-token chunks, block
permutation invariance, and planted mistakes that each pin must catch."""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.paged_attention as pa
from helpers import upcast
from paged_kv_cache_247_amd import workload as W


def sdpa_prefill(wl) -> np.ndarray:
    """Each sequence's new tokens against its logical K/V stream (fp64, CPU), with the mask
    that lets the token at position L - Q + t see positions 0 .. L - Q + t."""
    c = wl.cfg
    out = np.zeros((int(wl.query_start[-1]), c.num_heads, c.head_dim))
    for i in range(c.num_seqs):
        L, Q = int(wl.context_lens[i]), int(wl.query_lens[i])
        r0 = int(wl.query_start[i])
        if Q == 0:
            continue
        q = torch.from_numpy(upcast(wl.q_prefill[r0:r0 + Q], c.dtype)).permute(1, 0, 2)[None]
        K = torch.from_numpy(upcast(wl.logical_k[i], c.dtype)).permute(1, 0, 2)[None]
        V = torch.from_numpy(upcast(wl.logical_v[i], c.dtype)).permute(1, 0, 2)[None]
        pos = np.arange(L)[None, :]
        limit = (L - Q + np.arange(Q))[:, None]
        mask = torch.from_numpy(pos <= limit)
        o = F.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=c.scale,
                                           enable_gqa=c.num_heads != c.num_kv_heads)
        out[r0:r0 + Q] = o[0].permute(1, 0, 2).numpy()
    return out


def run_prefill(wl):
    c = wl.cfg
    return oracle.prefill(wl.q_prefill, wl.k_cache, wl.v_cache, wl.block_tables,
                          wl.context_lens, wl.query_start, c.scale, c.num_kv_heads, c.dtype)


def check_sdpa(wl) -> float:
    return float(np.abs(run_prefill(wl) - sdpa_prefill(wl)).max())


CASES = [("p1", {}), ("p2", {}), ("p1", {"num_heads": 2, "num_kv_heads": 2}),
         ("p1", {"block_size": 32, "dtype": "f32"}), ("p2", {"num_heads": 16})]


@pytest.mark.parametrize("name,over", CASES)
def test_prefill_equals_masked_sdpa(name, over):
    wl = W.generate(W.PREFILL_SMALL[name].replace(**over), keep_logical=True)
    assert check_sdpa(wl) < 1e-12


def test_whole_prompt_is_causal_self_attention():
    """Q = L: torch's own is_causal path (no hand-built mask)."""
    wl = W.generate(W.PREFILL_SMALL["p2"], keep_logical=True)
    c = wl.cfg
    got = run_prefill(wl)
    for i in range(c.num_seqs):
        L = int(wl.context_lens[i])
        r0 = int(wl.query_start[i])
        assert int(wl.query_lens[i]) == L
        q = torch.from_numpy(upcast(wl.q_prefill[r0:r0 + L], c.dtype)).permute(1, 0, 2)[None]
        K = torch.from_numpy(upcast(wl.logical_k[i], c.dtype)).permute(1, 0, 2)[None]
        V = torch.from_numpy(upcast(wl.logical_v[i], c.dtype)).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(q, K, V, is_causal=True, scale=c.scale,
                                           enable_gqa=True)
        assert np.abs(got[r0:r0 + L] - o[0].permute(1, 0, 2).numpy()).max() < 1e-12


def test_one_token_chunks_equal_decode():
    cfg = W.PREFILL_SMALL["p1"].replace(query_len=1)
    wl = W.generate(cfg)
    got = run_prefill(wl)
    ref = oracle.decode(wl.q_prefill, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                        cfg.scale, cfg.num_kv_heads, cfg.dtype)
    assert np.abs(got - ref).max() < 1e-13


def test_block_permutation_invariance():
    wl = W.generate(W.PREFILL_SMALL["p1"])
    a = run_prefill(wl)
    b = run_prefill(W.permute_pool(wl, 5))
    assert np.array_equal(a, b)


def test_work_items_cover_every_tile_once():
    wl = W.generate(W.PREFILL["p2"].replace(num_blocks=4096))
    for tile in (16, 64, 256):
        items = wl.prefill_work_items(tile)
        T = max(-(-int(wl.query_lens.max()) // tile), 1)
        want = {i * T + t for i in range(wl.cfg.num_seqs)
                for t in range(-(-int(wl.query_lens[i]) // tile))}
        assert sorted(items.tolist()) == sorted(want)
        cost = [int(wl.context_lens[u // T] - wl.query_lens[u // T])
                + min((u % T + 1) * tile, int(wl.query_lens[u // T])) for u in items]
        assert cost == sorted(cost, reverse=True)


def test_prefill_flops_closed_form():
    wl = W.generate(W.PREFILL_SMALL["p1"])
    c = wl.cfg
    pairs = sum(sum(int(L) - int(Q) + t + 1 for t in range(int(Q)))
                for L, Q in zip(wl.context_lens, wl.query_lens))
    assert wl.prefill_flops() == pairs * c.num_heads * c.head_dim * 4


# ---------------------------------------------------------------- planted mistakes

def _prefill_with_limit(shift, top_left=False):
    """A mutant that lets token t see positions 0 .. limit + shift (top_left: limit = t)."""
    def mutant(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
               num_kv_heads, dtype):
        T, H, D = q.shape
        G = H // num_kv_heads
        qf = pa.to_f64(q, dtype)
        out = np.zeros((T, H, D))
        for i in range(len(context_lens)):
            L = int(context_lens[i])
            r0, r1 = int(query_start[i]), int(query_start[i + 1])
            Q = r1 - r0
            for g in range(num_kv_heads):
                K, V = pa.gather(k_cache, v_cache, block_tables[i], L, g, k_cache.shape[2], dtype)
                for t in range(Q):
                    p = (t if top_left else L - Q + t) + shift
                    p = min(max(p, 0), L - 1)
                    for h in range(g * G, (g + 1) * G):
                        out[r0 + t, h] = pa._attend(qf[r0 + t, h], K[:p + 1], V[:p + 1], scale)
        return out
    return mutant


@pytest.mark.parametrize("mutant", [_prefill_with_limit(-1), _prefill_with_limit(+1),
                                    _prefill_with_limit(0, top_left=True)],
                         ids=["excludes-self", "sees-next", "top-left-aligned"])
def test_planted_mistake_fails_the_sdpa_pin(monkeypatch, mutant):
    monkeypatch.setattr(oracle, "prefill", mutant)
    wl = W.generate(W.PREFILL_SMALL["p1"], keep_logical=True)
    assert check_sdpa(wl) > 1e-6
