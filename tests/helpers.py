"""Shared test helpers: golden-fixture loading and library-routine cross-checks.

Nothing here computes paged attention itself; the cross-checks below call torch's
scaled_dot_product_attention on contiguous (dense) tensors built from the generator's logical
K/V stream, never from the pool.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(x):
    if isinstance(x, str):
        if x == "nan":
            return math.nan
        return float(Fraction(x))
    return float(x)


def golden_array(nested) -> np.ndarray:
    """Nested lists of numbers / "nan" / "p/q" strings -> float64 array."""
    def conv(v):
        return [conv(e) for e in v] if isinstance(v, list) else _num(v)
    return np.array(conv(nested), dtype=np.float64)


def load_golden(name="decode_closed_form.json"):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def upcast(a: np.ndarray, dtype: str) -> np.ndarray:
    """Test-side upcast of stored elements (independent of the oracle's)."""
    if dtype == "bf16":
        return torch.from_numpy(a.astype(np.int16).copy()).view(torch.bfloat16).double().numpy()
    return a.astype(np.float64)


def dense_sdpa(wl) -> np.ndarray:
    """Conventional padded batch: K/V contiguous per sequence, padded to the longest context
    and masked beyond each length; torch's SDPA (fp64, CPU) with grouped-query expansion."""
    c = wl.cfg
    B, H, D, Hkv = c.num_seqs, c.num_heads, c.head_dim, c.num_kv_heads
    Lmax = max(int(wl.context_lens.max()), 1)
    K = np.zeros((B, Hkv, Lmax, D))
    V = np.zeros((B, Hkv, Lmax, D))
    mask = np.zeros((B, 1, 1, Lmax), dtype=bool)
    for i in range(B):
        L = int(wl.context_lens[i])
        K[i, :, :L] = upcast(wl.logical_k[i], c.dtype).transpose(1, 0, 2)
        V[i, :, :L] = upcast(wl.logical_v[i], c.dtype).transpose(1, 0, 2)
        mask[i, ..., :L] = True
    q = torch.from_numpy(upcast(wl.q, c.dtype)).unsqueeze(2)  # [B, H, 1, D]
    out = F.scaled_dot_product_attention(q, torch.from_numpy(K), torch.from_numpy(V),
                                         attn_mask=torch.from_numpy(mask), scale=c.scale,
                                         enable_gqa=(H != Hkv))
    out = out.squeeze(2).numpy().copy()
    out[wl.context_lens == 0] = 0.0
    return out


def causal_last_rows(wl, seed=7) -> np.ndarray:
    """Full recompute: causal self-attention over each whole sequence with the decode query
    as the last query row; the last output row is what cached decode must return."""
    c = wl.cfg
    rng = np.random.default_rng(seed)
    out = np.zeros((c.num_seqs, c.num_heads, c.head_dim))
    for i in range(c.num_seqs):
        L = int(wl.context_lens[i])
        Q = rng.standard_normal((c.num_heads, L, c.head_dim))
        Q[:, -1, :] = upcast(wl.q[i], c.dtype)
        K = upcast(wl.logical_k[i], c.dtype).transpose(1, 0, 2)
        V = upcast(wl.logical_v[i], c.dtype).transpose(1, 0, 2)
        o = F.scaled_dot_product_attention(torch.from_numpy(Q)[None], torch.from_numpy(K)[None],
                                           torch.from_numpy(V)[None], is_causal=True,
                                           scale=c.scale, enable_gqa=(c.num_heads != c.num_kv_heads))
        out[i] = o[0, :, -1, :].numpy()
    return out
