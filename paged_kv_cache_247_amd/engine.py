"""A live decode loop over the paged kernels: an iteration-level scheduler on top of the block
manager, on synthetic tokens.

Continuous batching as the Qualiteg post describes it ("In a Nutshell ..." item 2-2): the
batch is re-formed at every iteration instead of per request, so requests join as soon as
their blocks fit, leave the moment they finish, and are swapped out to host memory and back
when the pool runs short (item 1-3: blocks are taken and returned as needed). Requests that
share a prefix share its blocks and get private copies of a shared block when they write into
it (Hacker News discussion of PagedAttention).

With prefill_chunk > 0 prompts are not written whole at admission: each step a prompting
sequence takes its next chunk of up to prefill_chunk prompt tokens (their K/V written, then one
paged prefill launch gives every chunk token's attention output over the sequence so far) while
the other sequences decode, so long prompts do not stall the batch.

There is no model: the query, key and value vectors of position p of request r are seeded
draws (N(0,1) rounded to the cache type), so that every step's attention can be checked
against a plain reference over each sequence's history. Each step is: swap-ins, admissions
(the prompt's K/V written with reshape_and_cache), one slot per running sequence (copy-on-write
block copies first; preemption by swap-out when blocks run out), then one decode launch that
also writes every sequence's newest K/V. Everything runs on the current stream in that order.
"""
from __future__ import annotations

import dataclasses
from collections import deque

import numpy as np
import torch

from . import _lib as L
from . import sharing
from .workload import cast_from_f32

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass
class Request:
    rid: int
    prompt_len: int
    new_tokens: int       # tokens to generate
    generated: int = 0
    origin: int = -1      # request whose stream this one continues (forks), -1 = its own
    fork_pos: int = 0     # positions inherited from origin
    prefilled: int = 0    # prompt positions in the cache (chunked prefill)


class DecodeEngine:
    def __init__(self, num_blocks: int, num_host_blocks: int, num_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, max_blocks_per_seq: int, dtype: str = "bf16",
                 seed: int = 0, prefill_chunk: int = 0, device="cuda", ops=None,
                 share_prefixes: bool = False):
        """ops: the kernel entry points (reshape_and_cache, copy_blocks, swap_blocks,
        paged_attention, paged_attention_prefill, paged_attention_shared); the HIP library by
        default. The block manager is always the library's. share_prefixes: decode sequences
        whose tables share leading blocks (forks) through shared-prefix groups, which read a
        shared tile once per group (sharing.plan)."""
        self.H, self.Hkv, self.D, self.S = num_heads, num_kv_heads, head_dim, block_size
        self.MB, self.dtype, self.seed = max_blocks_per_seq, dtype, seed
        self.chunk = prefill_chunk
        self.share = share_prefixes
        self.scale = 1.0 / float(np.sqrt(head_dim))
        self.ops = ops if ops is not None else L
        self.device = torch.device(device)
        self.bm = L.BlockManager(num_blocks, num_host_blocks, block_size)
        tdt = _TORCH[dtype]
        self.k = torch.zeros((num_blocks, num_kv_heads, block_size, head_dim), dtype=tdt,
                             device=self.device)
        vshape = L.v_block_shape(num_kv_heads, head_dim, block_size)
        self.v = torch.zeros((num_blocks, *vshape), dtype=tdt, device=self.device)
        pin = self.device.type == "cuda"
        self.hk = torch.zeros((max(num_host_blocks, 1), num_kv_heads, block_size, head_dim),
                              dtype=tdt, pin_memory=pin)
        self.hv = torch.zeros((max(num_host_blocks, 1), *vshape), dtype=tdt, pin_memory=pin)
        self.requests: dict[int, Request] = {}
        self.waiting: deque[int] = deque()
        self.running: list[int] = []
        self.swapped: deque[int] = deque()
        self.finished: list[int] = []
        self.stats = {"steps": 0, "swap_outs": 0, "swap_ins": 0, "cow_copies": 0,
                      "admitted": 0, "prefill_chunks": 0, "short_chunks": 0, "shared_groups": 0}

    # ------------------------------------------------------------ synthetic tokens
    def _stream_owner(self, rid: int, pos: int) -> int:
        """Request whose stream holds position pos of rid (forks inherit their origin's)."""
        r = self.requests[rid]
        while r.origin >= 0 and pos < r.fork_pos:
            r = self.requests[r.origin]
        return r.rid

    def token(self, rid: int, pos: int):
        """(q [H, D], k [Hkv, D], v [Hkv, D]) of position pos of request rid, storage type."""
        owner = self._stream_owner(rid, pos)
        rng = np.random.default_rng([self.seed, owner, pos])
        x = rng.standard_normal((self.H + 2 * self.Hkv, self.D), dtype=np.float32)
        x = cast_from_f32(x, self.dtype)
        return x[:self.H], x[self.H:self.H + self.Hkv], x[self.H + self.Hkv:]

    def _dev(self, a: np.ndarray) -> torch.Tensor:
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(self.device)
        return torch.from_numpy(a).to(self.device)

    # ------------------------------------------------------------ requests
    def submit(self, rid: int, prompt_len: int, new_tokens: int):
        if rid in self.requests:
            raise ValueError(f"request id {rid} is taken")
        if prompt_len < 0 or new_tokens < 1:
            raise ValueError("prompt_len >= 0 and new_tokens >= 1")
        self.requests[rid] = Request(rid, prompt_len, new_tokens)
        self.waiting.append(rid)

    def fork(self, parent: int, child: int, new_tokens: int):
        """child continues parent's sequence as it stands, sharing its blocks; its own tokens
        start at the parent's current length."""
        if parent not in self.running:
            raise ValueError("only a running request can be forked")
        if self.requests[parent].prefilled < self.requests[parent].prompt_len:
            raise ValueError("a request still reading its prompt cannot be forked")
        if child in self.requests:
            raise ValueError(f"request id {child} is taken")
        if new_tokens < 1:
            raise ValueError("new_tokens >= 1")
        n = self.bm.num_tokens(parent)
        self.bm.fork(parent, child)
        self.requests[child] = Request(child, n, new_tokens, origin=parent, fork_pos=n,
                                       prefilled=n)
        self.running.append(child)

    # ------------------------------------------------------------ one iteration
    def _write_prompt(self, rid: int):
        n = self.requests[rid].prompt_len
        if n == 0:
            return
        t, _ = self.bm.tables([rid], self.MB)
        pos = np.arange(n)
        slots = t[0, pos // self.S].astype(np.int64) * self.S + pos % self.S
        toks = [self.token(rid, int(p)) for p in pos]
        ks = np.stack([k for _, k, _ in toks])
        vs = np.stack([v for _, _, v in toks])
        self.ops.reshape_and_cache(self._dev(ks), self._dev(vs), self.k, self.v, self._dev(slots))

    def _swap_out(self, rid: int):
        pairs = self.bm.swap_out(rid)
        self.ops.swap_blocks(self.k, self.v, self.hk, self.hv, pairs, to_device=False)
        self.running.remove(rid)
        self.swapped.appendleft(rid)
        self.stats["swap_outs"] += 1

    def _swap_in(self, rid: int):
        pairs = self.bm.swap_in(rid)
        self.ops.swap_blocks(self.hk, self.hv, self.k, self.v, pairs, to_device=True)
        self.running.append(rid)
        self.stats["swap_ins"] += 1

    def _prompting(self, rid: int) -> bool:
        r = self.requests[rid]
        return self.chunk > 0 and r.prefilled < r.prompt_len

    def step(self):
        """One iteration. Returns a dict: "decode" {rid: (row of decode_out, position)} with
        "decode_out" [B, H, D], and "prefill" {rid: (first row of prefill_out, first position,
        tokens)} with "prefill_out" [T, H, D] (outputs are None when nothing of that kind ran)."""
        # 1. swapped-out requests first (oldest preempted first), then new ones, while they fit
        while self.swapped:
            rid = self.swapped[0]
            need = -(-self.bm.num_tokens(rid) // self.S) + 1
            if self.bm.free_blocks < need:
                break
            self.swapped.popleft()
            self._swap_in(rid)
        while self.waiting and not self.swapped:
            rid = self.waiting[0]
            P = self.requests[rid].prompt_len
            first = min(self.chunk, P) if self.chunk else P
            if self.bm.free_blocks < -(-first // self.S) + 1:
                break
            self.waiting.popleft()
            if self.chunk:
                self.bm.add(rid, 0)
            else:
                self.bm.add(rid, P)
                self._write_prompt(rid)
                self.requests[rid].prefilled = P
            self.running.append(rid)
            self.stats["admitted"] += 1
        # 2. slots, in admission order: the next prompt chunk of a prompting sequence, one
        # token of a decoding one. When blocks run out, the youngest sequence that has not
        # taken its slots yet is swapped out (possibly the one asking) and the append is tried
        # again; a prompt chunk that got some of its slots is cut short instead.
        copies, order, i, take = [], list(self.running), 0, {}
        while i < len(order):
            rid = order[i]
            want = (min(self.chunk, self.requests[rid].prompt_len - self.requests[rid].prefilled)
                    if self._prompting(rid) else 1)
            got = 0
            try:
                while got < want:
                    _, cow = self.bm.append(rid)
                    got += 1
                    if cow is not None:
                        copies.append(cow)
            except L.OutOfBlocks:
                if got == 0:
                    if len(order) == 1:
                        raise
                    self._swap_out(order.pop())
                    continue
                self.stats["short_chunks"] += 1
            take[rid] = got
            i += 1
        if copies:
            self.ops.copy_blocks([self.k], [self.v], self._dev(np.asarray(copies, dtype=np.int64)))
            self.stats["cow_copies"] += len(copies)
        res = {"decode": {}, "decode_out": None, "prefill": {}, "prefill_out": None}
        pre = [r for r in order if self._prompting(r)]
        dec = [r for r in order if not self._prompting(r)]
        # 3. prompt chunks: their K/V into the cache, then causal attention of each chunk token
        # over its sequence so far
        if pre:
            t, lens = self.bm.tables(pre, self.MB)
            rows, slots, qs = [], [], [0]
            for r, tab, n in zip(pre, t, lens):
                p0 = self.requests[r].prefilled
                for p in range(p0, int(n)):
                    rows.append(self.token(r, p))
                    slots.append(int(tab[p // self.S]) * self.S + p % self.S)
                res["prefill"][r] = (qs[-1], p0, int(n) - p0)
                qs.append(qs[-1] + int(n) - p0)
            q = np.stack([x[0] for x in rows])
            self.ops.reshape_and_cache(self._dev(np.stack([x[1] for x in rows])),
                                self._dev(np.stack([x[2] for x in rows])), self.k, self.v,
                                self._dev(np.asarray(slots, dtype=np.int64)))
            out = torch.empty((len(rows), self.H, self.D), dtype=_TORCH[self.dtype],
                              device=self.device)
            self.ops.paged_attention_prefill(out, self._dev(q), self.k, self.v, self._dev(t),
                                      self._dev(lens), self._dev(np.asarray(qs, np.int32)),
                                      int(np.diff(qs).max()), self.scale)
            res["prefill_out"] = out
            for r, n in zip(pre, lens):
                self.requests[r].prefilled = int(n)
            self.stats["prefill_chunks"] += len(pre)
        # 4. decode every other running sequence, writing its newest K/V
        if dec:
            t, lens = self.bm.tables(dec, self.MB)
            toks = [self.token(r, int(n) - 1) for r, n in zip(dec, lens)]
            out = torch.empty((len(dec), self.H, self.D), dtype=_TORCH[self.dtype],
                              device=self.device)
            q = self._dev(np.stack([x[0] for x in toks]))
            nk = self._dev(np.stack([x[1] for x in toks]))
            nv = self._dev(np.stack([x[2] for x in toks]))
            plan = (sharing.plan(t, lens, self.S, int(lens.max()), self.H // self.Hkv)
                    if self.share else None)
            if plan is not None:
                self.ops.paged_attention_shared(
                    out, q, self.k, self.v, self._dev(t), self._dev(lens), int(lens.max()),
                    self.scale, self._dev(plan.groups), self._dev(plan.work_items),
                    plan.partition_size, new_key=nk, new_value=nv)
                self.stats["shared_groups"] += len(plan.groups)
            else:
                self.ops.paged_attention(out, q, self.k, self.v, self._dev(t), self._dev(lens),
                                         int(lens.max()), self.scale, 0, new_key=nk,
                                         new_value=nv)
            res["decode"] = {r: (k, int(n) - 1) for k, (r, n) in enumerate(zip(dec, lens))}
            res["decode_out"] = out
            # 5. finish
            for r in dec:
                req = self.requests[r]
                req.generated += 1
                if req.generated >= req.new_tokens:
                    self.bm.free(r)
                    self.running.remove(r)
                    self.finished.append(r)
        self.stats["steps"] += 1
        return res

    def done(self) -> bool:
        return not (self.waiting or self.running or self.swapped)
