"""Oracle for paged decode: a plain, slow CPU implementation in numpy float64.

TEST INFRASTRUCTURE. Only the tests, the smoke entry point and the CPU-baseline leg of the
benchmark may import or call this module. The product path never routes through it, and it
shares no code with the HIP library: it reads the pool layout from its written statement
(below) and does its own indexing, upcasting and arithmetic.

What is computed, and where each step comes from:

* Attention of one query token over its context. The attention operator takes K and V and
  the vAttention paper ("3 Issues with the PagedAttention Model", section 3.1 "Requires
  re-writing the attention kernel") names it but its equation is not on the page. The
  reading used here is the plain scaled-dot-product form out = softmax(scale * q K^T) V,
  with every cached position visible to the newest query (no mask, no positional term).
* The KV cache is split into fixed-size blocks placed anywhere in a physical pool, and a
  block table links each sequence's logical blocks to physical ones (Qualiteg, "About
  PagedAttention for LLM serving", "Deepening Our Understanding ..." item 1-2 and "There are
  logical blocks and physical blocks ... linked by a block table"). Paging changes where
  the bytes live, not the result, so the oracle gathers each sequence's blocks into
  contiguous K, V and then applies the plain definition.
* The batch is ragged with no padding (same post, "In a Nutshell ..." item 2-1): each
  sequence uses exactly its own context_lens[i] positions.
* Grouped-query attention (named in the vAttention section 3.1 text): consecutive query
  heads share one kv head, g = h // (H / Hkv).
* New K/V of each step are written into the cache (the cached generation loop of the
  Qualiteg post: only the new token is computed, the cache is updated each step); a slot
  is block_id * S + offset.
* Requests that share a prefix share its KV blocks (Hacker News discussion of
  PagedAttention, replies on prefix sharing); a private copy of a shared block
  (copy-on-write) copies every element of the block.
* Prefill: the first forward pass over the prompt computes every prompt token's output and
  fills the cache, after which generation feeds one token at a time (Qualiteg post,
  "Deepening Our Understanding ...", the past_key_values loop). A chunk of Q new tokens at the
  end of a sequence of L positions is the same computation: the token at position p attends
  to positions 0..p (causal), the whole prompt being the case Q = L.
* Split-context partitions and their merge are not on the pages; they are an exact
  rewriting of the softmax sum: per partition p, m_p = max logit, l_p = sum exp(s - m_p),
  o_p = sum exp(s - m_p) v / l_p; then M = max m_p, w_p = l_p exp(m_p - M),
  out = sum w_p o_p / sum w_p.

Layout (the same statement the C header makes; the pages fix none of it):
  q, out       [B, H, D]
  k_cache      [N, Hkv, S, D]   element (b, g, t, d)
  v_cache      [N, Hkv, (S / VS) D, VS] with VS = min(S, 32): position t of the block is
               column t % VS of column group t // VS, and head dim d is row d of that group,
               so element (b, g, d, t) sits at [b, g, (t // VS) D + d, t % VS]. For S <= 32
               there is one group and this is [N, Hkv, D, S].
  block_tables [B, MB] int32; entries past ceil(L_i / S) are never read
  context_lens [B] int32; L_i = 0 gives a zero output and no partials
bf16 arrays are uint16 bit patterns; "f64" storage is accepted for invariance tests.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["V_GROUP", "v_group", "to_f64", "write_cache", "copy_blocks", "gather", "decode", "decode_partials",
           "reduce_partials", "num_partitions", "prefill", "v_from_rows", "v_to_rows"]


V_GROUP = 32  # most block positions in one column group of the V layout


def v_group(block_size: int) -> int:
    """Positions per column group of a V block (VS in the layout statement)."""
    return min(int(block_size), V_GROUP)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored elements to float64."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f16", "f64"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(dtype)


def v_from_rows(v_rows, block_size):
    """The column-group V pool holding the same elements as a pool of token rows
    [N, Hkv, S, D] (the layout statement above, position by position)."""
    N, Hkv, S, D = v_rows.shape
    assert S == block_size
    VS = v_group(S)
    v = np.zeros((N, Hkv, S // VS * D, VS), dtype=v_rows.dtype)
    for t in range(S):
        v[:, :, (t // VS) * D:(t // VS + 1) * D, t % VS] = v_rows[:, :, t, :]
    return v


def v_to_rows(v_cache, block_size):
    """Token rows [N, Hkv, S, D] of a column-group V pool (the inverse of v_from_rows)."""
    N, Hkv, R, VS = v_cache.shape
    S = block_size
    assert VS == v_group(S) and R % (S // VS) == 0
    D = R // (S // VS)
    rows = np.zeros((N, Hkv, S, D), dtype=v_cache.dtype)
    for t in range(S):
        rows[:, :, t, :] = v_cache[:, :, (t // VS) * D:(t // VS + 1) * D, t % VS]
    return rows


def write_cache(k_cache, v_cache, key, value, slot_mapping, block_size):
    """Copies of the pools with each new token's K/V stored at its slot (bit copies).

    Token t with slot s >= 0 lands at block s // S, position s % S; a negative slot is
    skipped. Slots must be distinct (one correct result only then)."""
    S = block_size
    VS = v_group(S)
    D = k_cache.shape[3]
    slots = [int(s) for s in slot_mapping]
    live = [s for s in slots if s >= 0]
    assert len(set(live)) == len(live), "duplicate slots"
    k = k_cache.copy()
    v = v_cache.copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, off = s // S, s % S
        assert 0 <= b < k.shape[0], "slot outside the pool"
        grp, col = off // VS, off % VS
        for g in range(k.shape[1]):
            k[b, g, off, :] = key[t, g, :]
            v[b, g, grp * D:(grp + 1) * D, col] = value[t, g, :]
    return k, v


def copy_blocks(k_caches, v_caches, block_mapping):
    """Copies of every layer's pools with block dst := block src for each (src, dst) pair."""
    pairs = [(int(s), int(d)) for s, d in np.asarray(block_mapping).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts), "repeated destination"
    assert not set(dsts) & {s for s, _ in pairs}, "a destination is also a source"
    ks = [k.copy() for k in k_caches]
    vs = [v.copy() for v in v_caches]
    for k, v in zip(ks, vs):
        for s, d in pairs:
            k[d] = k[s]
            v[d] = v[s]
    return ks, vs


def gather(k_cache, v_cache, table_row, L, g, block_size, dtype):
    """Contiguous K_i, V_i [L, D] (float64) of one sequence and kv head g."""
    S = block_size
    VS = v_group(S)
    D = k_cache.shape[3]
    nb = -(-int(L) // S)
    Ks, Vs = [], []
    for j in range(nb):
        b = int(table_row[j])
        assert 0 <= b < k_cache.shape[0], "block id outside the pool"
        rows = min(S, int(L) - j * S)
        Ks.append(to_f64(k_cache[b, g, :rows, :], dtype))
        # V positions 0..rows-1 of the block, column group by column group
        for grp in range(-(-rows // VS)):
            cols = min(VS, rows - grp * VS)
            Vs.append(to_f64(v_cache[b, g, grp * D:(grp + 1) * D, :cols], dtype).T)
    if not Ks:
        return np.zeros((0, D)), np.zeros((0, D))
    return np.concatenate(Ks, axis=0), np.concatenate(Vs, axis=0)


def _attend(qv, K, V, scale):
    s = scale * (K @ qv)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, dtype):
    """out[i, h] = softmax(scale * q[i, h] K_i^T) V_i over the L_i gathered positions of
    kv head h // G; zero when L_i = 0. Returns float64 [B, H, D]."""
    B, H, D = q.shape
    G = H // num_kv_heads
    assert G * num_kv_heads == H
    S = k_cache.shape[2]
    qf = to_f64(q, dtype)
    out = np.zeros((B, H, D))
    for i in range(B):
        L = int(context_lens[i])
        if L == 0:
            continue
        for g in range(num_kv_heads):
            K, V = gather(k_cache, v_cache, block_tables[i], L, g, S, dtype)
            for h in range(g * G, (g + 1) * G):
                out[i, h] = _attend(qf[i, h], K, V, scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
            num_kv_heads, dtype):
    """Causal attention of each sequence's new tokens over its cache.

    Sequence i has Q_i = query_start[i + 1] - query_start[i] new tokens, rows
    query_start[i] .. query_start[i + 1] - 1 of q [T, H, D], at positions L_i - Q_i .. L_i - 1
    (L_i = context_lens[i], the cache holding all L_i positions). The token at position p and
    head h gets softmax(scale * q K_i[0..p]^T) V_i[0..p] over kv head h // G. Returns float64
    [T, H, D]."""
    T, H, D = q.shape
    G = H // num_kv_heads
    assert G * num_kv_heads == H
    S = k_cache.shape[2]
    qf = to_f64(q, dtype)
    out = np.zeros((T, H, D))
    for i in range(len(context_lens)):
        L = int(context_lens[i])
        r0, r1 = int(query_start[i]), int(query_start[i + 1])
        Q = r1 - r0
        assert 0 <= Q <= L, "more new tokens than positions"
        for g in range(num_kv_heads):
            K, V = gather(k_cache, v_cache, block_tables[i], L, g, S, dtype)
            for t in range(Q):
                p = L - Q + t
                for h in range(g * G, (g + 1) * G):
                    out[r0 + t, h] = _attend(qf[r0 + t, h], K[:p + 1], V[:p + 1], scale)
    return out


def num_partitions(L, partition_size):
    return -(-int(L) // partition_size)


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads,
                    dtype, partition_size, max_partitions=None):
    """Per-partition (m_p, l_p, o_p) of every (sequence, head).

    Partition p covers positions [p P, min((p+1) P, L_i)). m_p is the max logit, l_p the sum
    of exp(s - m_p), o_p the normalised partial output. Entries of partitions p >= ceil(L_i/P)
    are NaN (never written)."""
    B, H, D = q.shape
    G = H // num_kv_heads
    S = k_cache.shape[2]
    P = int(partition_size)
    NPmax = max_partitions or max([num_partitions(L, P) for L in context_lens] + [1])
    qf = to_f64(q, dtype)
    m = np.full((B, H, NPmax), np.nan)
    l = np.full((B, H, NPmax), np.nan)
    o = np.full((B, H, NPmax, D), np.nan)
    for i in range(B):
        L = int(context_lens[i])
        for g in range(num_kv_heads):
            K, V = gather(k_cache, v_cache, block_tables[i], L, g, S, dtype)
            for h in range(g * G, (g + 1) * G):
                s = scale * (K @ qf[i, h])
                for p in range(num_partitions(L, P)):
                    sp = s[p * P:(p + 1) * P]
                    mp = sp.max()
                    e = np.exp(sp - mp)
                    m[i, h, p] = mp
                    l[i, h, p] = e.sum()
                    o[i, h, p] = (e @ V[p * P:(p + 1) * P]) / e.sum()
    return m, l, o


def reduce_partials(m, l, o, context_lens, partition_size):
    """Merge partitions: M = max m_p, w_p = l_p exp(m_p - M), out = sum w_p o_p / sum w_p."""
    B, H, _, D = o.shape
    out = np.zeros((B, H, D))
    for i in range(B):
        n = num_partitions(context_lens[i], partition_size)
        if n == 0:
            continue
        for h in range(H):
            M = m[i, h, :n].max()
            w = l[i, h, :n] * np.exp(m[i, h, :n] - M)
            out[i, h] = (w @ o[i, h, :n]) / w.sum()
    return out


def max_abs_err(gpu, ref):
    """max |gpu - ref| over all elements (inf if either side has a NaN where the other not)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    if gpu.shape != ref.shape:
        raise ValueError(f"shape {gpu.shape} vs {ref.shape}")
    if gpu.size == 0:
        return 0.0
    d = np.abs(gpu - ref)
    if np.isnan(d).any():
        return math.inf
    return float(d.max())
