"""Plain CPU model of the KV-cache control plane (test infrastructure only).

Follows the BlockManager the pages describe (“Nano-vLLM 引擎架构解析”, section 3.2
"PagedAttention"; “深入 Nano-vLLM 推理引擎”, headings "Handling resource exhaustion",
"From Sequences to Blocks", "Prefix Caching by hashing", "Control plane vs.
data plane"):

* a ``Block`` carries an id, a reference count and its token ids;
* the manager keeps a deque of free blocks and a map of used ones and hands out
  the free block at the head of the deque;
* a sequence is cut into fixed-size blocks, never sharing a block with another
  sequence except for a shared prefix, whose block ids are reused with their
  reference counts raised;
* freeing only marks a block free: its GPU contents are not cleared.

Reading where the pages disagree: the printed ``allocate`` invents a new block id
when the free deque is empty, which would grow a fixed pool without bound and
clash with live ids; here the pool is fixed and allocation fails (returns None),
which is when the scheduler preempts a sequence.  A freed block goes to the tail
of the free deque.

``plan_step`` turns a workload into the per-step metadata the data plane needs:
block tables, the slot of every token written, cumulative sequence lengths for
prefill ("Preparing for computation") and context lengths for decode.
"""
from __future__ import annotations

from collections import deque

import numpy as np

__all__ = ["Block", "BlockManager", "PrefixCache", "slot_of", "cumulative_lengths", "plan_step"]


class Block:
    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_count = 0
        self.token_ids = []


class BlockManager:
    def __init__(self, num_blocks: int, free_order=None):
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        self.blocks = [Block(i) for i in range(num_blocks)]
        self.free_blocks = deque(order)
        self.used_blocks = {}

    def allocate(self):
        """Head of the free deque, reference count 1; None when the pool is empty."""
        if not self.free_blocks:
            return None
        block_id = self.free_blocks.popleft()
        block = self.blocks[block_id]
        block.ref_count = 1
        block.token_ids = []
        self.used_blocks[block_id] = block
        return block_id

    def share(self, block_id: int) -> None:
        """Reuse a cached block: one more reference, no copy."""
        self.used_blocks[block_id].ref_count += 1

    def free(self, block_id: int) -> None:
        """Drop one reference; at zero the block returns to the free deque (not cleared)."""
        block = self.used_blocks[block_id]
        block.ref_count -= 1
        if block.ref_count == 0:
            del self.used_blocks[block_id]
            self.free_blocks.append(block_id)


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

    Sequences take blocks from the free deque in index order; a sequence in a
    prefix group other than the group's first reuses the first one's prefix
    blocks (``share``) and allocates the rest.  Returns plain Python lists:

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
    mgr = BlockManager(wl.num_blocks, wl.free_order)
    tables = []
    group_owner = {}
    for i, s in enumerate(wl.seqs):
        n_blocks = -(-s.context_len // bs)
        table = []
        if s.prefix_group >= 0 and s.prefix_group in group_owner:
            owner_table = tables[group_owner[s.prefix_group]]
            for j in range(s.prefix_len // bs):
                mgr.share(owner_table[j])
                table.append(owner_table[j])
        elif s.prefix_group >= 0:
            group_owner[s.prefix_group] = i
        while len(table) < n_blocks:
            b = mgr.allocate()
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
        "ref_counts": {b: blk.ref_count for b, blk in mgr.used_blocks.items()},
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
