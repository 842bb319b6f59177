"""Plain CPU model of the KV-cache control plane (test infrastructure only).

What the pages say the control plane does (“Nano-vLLM 引擎架构解析”, section 3.2
"PagedAttention"; “深入 Nano-vLLM 推理引擎”, headings "Handling resource exhaustion",
"From Sequences to Blocks", "Prefix Caching by hashing", "Control plane vs. data
plane"), modelled as directly as possible:

* the KV pool is a fixed set of block ids; each id has a reference count, zero
  meaning the block is free;
* free ids wait in a first-in first-out queue and a request takes the oldest one;
* a sequence's tokens fill its own blocks in order, except that a cached prefix is
  reused by listing the same ids again, each reuse adding one reference;
* releasing a reference that was the last one puts the id back at the end of the
  queue; the block's GPU contents are left as they are.

Reading where the pages disagree: the printed allocation routine makes up a new id
when nothing is free, which would grow a fixed pool and collide with live ids; here
a request on an empty queue fails (``take`` returns None), which is the point where
the scheduler preempts a sequence.

``plan_step`` turns a workload into the per-step metadata the data plane needs:
block tables, the slot of every token written, cumulative sequence lengths for
prefill ("Preparing for computation") and context lengths for decode.
"""
from __future__ import annotations

from collections import deque

import numpy as np

__all__ = ["IdPool", "PrefixCache", "slot_of", "cumulative_lengths", "plan_step"]


class IdPool:
    """Block ids 0 .. num_blocks-1 with reference counts and a queue of free ids
    (initially ``free_order``, else id order)."""

    def __init__(self, num_blocks: int, free_order=None):
        self.refs = [0] * num_blocks
        self.free_ids = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]

    def take(self):
        """The oldest free id with one reference, or None when every id is in use."""
        if len(self.free_ids) == 0:
            return None
        b = self.free_ids.pop(0)
        self.refs[b] = 1
        return b

    def retain(self, b: int) -> None:
        """One more reference to an id in use (a shared cached block; nothing copied)."""
        assert self.refs[b] > 0, "retain of a free block"
        self.refs[b] += 1

    def release(self, b: int) -> None:
        """One reference fewer; the last one sends the id to the back of the queue."""
        assert self.refs[b] > 0, "release of a free block"
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free_ids.append(b)

    def in_use(self) -> dict:
        """{id: reference count} of every id in use."""
        return {b: r for b, r in enumerate(self.refs) if r > 0}


def slot_of(table_row, position: int, block_size: int) -> int:
    """Token ``position`` of a sequence lives in block table_row[position // block_size]
    at offset position % block_size; its slot is block * block_size + offset."""
    return int(table_row[position // block_size]) * block_size + position % block_size


def cumulative_lengths(lengths) -> list:
    """[0, l0, l0+l1, ...]."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


def plan_step(wl, table_pad: int = -1) -> dict:
    """Allocate every sequence's blocks in order and build the step's metadata.

    Sequences take blocks from the free queue in index order; a sequence in a
    prefix group other than the group's first reuses the first one's prefix
    blocks (``retain``) and takes the rest.  Returns plain Python lists:

    tables            per sequence, its block ids
    history_slots     (seq, position, slot) of tokens written before the step
    step_slots        (seq, position, slot) of the step's new tokens
    prefill / decode  index lists of the sequences in each phase
    cu_seqlens_q/k    over the prefill sequences
    context_lens      over the decode sequences
    block_tables      prefill and decode tables padded with ``table_pad`` to the
                      widest table of the step
    """
    bs = wl.block_size
    pool = IdPool(wl.num_blocks, wl.free_order)
    tables = []
    group_owner = {}
    for i, s in enumerate(wl.seqs):
        n_blocks = -(-s.context_len // bs)
        table = []
        if s.prefix_group >= 0 and s.prefix_group in group_owner:
            owner_table = tables[group_owner[s.prefix_group]]
            for j in range(s.prefix_len // bs):
                pool.retain(owner_table[j])
                table.append(owner_table[j])
        elif s.prefix_group >= 0:
            group_owner[s.prefix_group] = i
        while len(table) < n_blocks:
            b = pool.take()
            if b is None:
                raise RuntimeError("pool exhausted")
            table.append(b)
        tables.append(table)

    history, step = [], []
    for i, s in enumerate(wl.seqs):
        first = s.prefix_len if (s.prefix_group >= 0 and group_owner[s.prefix_group] != i) else 0
        for p in range(first, s.history_len):
            history.append((i, p, slot_of(tables[i], p, bs)))
        for p in range(s.history_len, s.context_len):
            step.append((i, p, slot_of(tables[i], p, bs)))

    prefill = wl.prefill_seqs
    decode = wl.decode_seqs
    width = max([len(t) for t in tables] + [1])

    def padded(idx):
        return [tables[i] + [table_pad] * (width - len(tables[i])) for i in idx]

    return {
        "tables": tables,
        "ref_counts": pool.in_use(),
        "history_slots": history,
        "step_slots": step,
        "prefill": prefill,
        "decode": decode,
        "cu_seqlens_q": cumulative_lengths(wl.seqs[i].new_tokens for i in prefill),
        "cu_seqlens_k": cumulative_lengths(wl.seqs[i].context_len for i in prefill),
        "context_lens": [wl.seqs[i].context_len for i in decode],
        "prefill_block_tables": padded(prefill),
        "decode_block_tables": padded(decode),
        "table_width": width,
    }


class PrefixCache:
    """Plain model of the prefix-cached block manager (test infrastructure only).

    “深入 Nano-vLLM 推理引擎”, "Prefix Caching by hashing": the manager maps the hash of a
    block to its id; a new sequence whose block is found takes it with one more
    reference.  Here the map is keyed by the exact thing a chained block hash stands
    for - the whole token prefix up to the end of the block - so the model needs no
    hash function and has no collisions.  Readings (the pages are silent on them):

    * only full blocks are cached; the last partial block is always new;
    * lookups run from the first block and stop at the first miss (a prefix cache
      reuses a cached prefix, not blocks after a gap);
    * a new full block is registered at once; a block handed out again loses its
      old registration, so stale contents are never a hit;
    * a cached block that was freed (reference count 0) but not handed out again is
      taken back off the free deque on a hit;
    * a sequence's blocks are freed last block first, to the tail of the free deque;
    * allocation and append are all-or-nothing when too few blocks are free.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        self.bs = int(block_size)
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.key_of = [None] * num_blocks   # the prefix a block is registered under
        self.by_key = {}                    # prefix tuple -> block id
        self.seqs = {}
        self.next_id = 0

    def add_sequence(self, tokens) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = {"tokens": [int(t) for t in tokens], "table": [], "cached": 0}
        return sid

    def _plan(self, toks):
        bs = self.bs
        hits = []
        for j in range(len(toks) // bs):
            b = self.by_key.get(tuple(toks[:(j + 1) * bs]))
            if b is None:
                break
            hits.append(b)
        n_blocks = -(-len(toks) // bs)
        takes = (n_blocks - len(hits)) + sum(1 for b in hits if self.ref[b] == 0)
        return hits, takes

    def can_allocate(self, sid) -> bool:
        return self._plan(self.seqs[sid]["tokens"])[1] <= len(self.free)

    def _take(self):
        b = self.free.popleft()
        if self.key_of[b] is not None:
            if self.by_key.get(self.key_of[b]) == b:
                del self.by_key[self.key_of[b]]
            self.key_of[b] = None
        self.ref[b] = 1
        return b

    def _register(self, b, key):
        old = self.by_key.get(key)
        if old is not None and old != b:
            self.key_of[old] = None
        self.by_key[key] = b
        self.key_of[b] = key

    def allocate(self, sid) -> bool:
        s = self.seqs[sid]
        if s["table"]:
            raise ValueError("sequence already holds blocks")
        toks, bs = s["tokens"], self.bs
        hits, takes = self._plan(toks)
        if takes > len(self.free):
            return False
        table = []
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
                self.ref[b] = 1
            else:
                self.ref[b] += 1
            table.append(b)
        for j in range(len(hits), len(toks) // bs):
            b = self._take()
            self._register(b, tuple(toks[:(j + 1) * bs]))
            table.append(b)
        if len(toks) % bs:
            table.append(self._take())
        s["table"], s["cached"] = table, len(hits) * bs
        return True

    def can_append(self, sid) -> bool:
        return len(self.seqs[sid]["tokens"]) % self.bs != 0 or len(self.free) > 0

    def append_token(self, sid, token) -> bool:
        s = self.seqs[sid]
        n = len(s["tokens"])
        if n % self.bs == 0:
            if not self.free:
                return False
            s["table"].append(self._take())
        s["tokens"].append(int(token))
        if (n + 1) % self.bs == 0:
            self._register(s["table"][-1], tuple(s["tokens"]))
        return True

    def deallocate(self, sid) -> None:
        s = self.seqs[sid]
        for b in reversed(s["table"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        s["table"], s["cached"] = [], 0

    def remove_sequence(self, sid) -> None:
        self.deallocate(sid)
        del self.seqs[sid]
