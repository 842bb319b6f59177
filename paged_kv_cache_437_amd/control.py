"""Control plane: the KV block pool and the per-step device metadata.

The pages put block bookkeeping on the CPU and KV data on the GPU (“深入 Nano-vLLM 推理引擎”,
"Control plane vs. data plane"): the pool hands out fixed-size blocks
(256 tokens by default, “Nano-vLLM 引擎架构解析” section 3.2) from the head of a
free list, counts references so that sequences with a common prefix reuse the
same block ids ("Prefix Caching by hashing"), and on release only marks a block
free - its device contents stay until a later write overwrites them.  When no
block is left, allocation fails and the scheduler preempts a sequence
("Handling resource exhaustion"); the pool never grows.

``plan_step`` turns a batch of sequences into what the kernels read: block
tables, the slot of every token written, cumulative lengths for prefill
("Preparing for computation") and context lengths for decode.  Arrays are
int32 numpy, built with vector operations; ``DeviceStep`` in ``step.py`` moves
them to the device.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

__all__ = ["BlockPool", "StepPlan", "plan_step", "slots_of_positions"]


class BlockPool:
    """Fixed pool of ``num_blocks`` KV blocks with reference counts."""

    def __init__(self, num_blocks: int, free_order=None):
        self.num_blocks = int(num_blocks)
        order = np.arange(num_blocks) if free_order is None else np.asarray(free_order)
        if sorted(order.tolist()) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool's ids")
        self._free = deque(int(b) for b in order)
        self.ref = np.zeros(num_blocks, np.int32)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self):
        """A free block with one reference, or None when the pool is exhausted."""
        if not self._free:
            return None
        b = self._free.popleft()
        self.ref[b] = 1
        return b

    def allocate_many(self, n: int):
        """``n`` blocks, or None (and nothing taken) if fewer are free."""
        if n > len(self._free):
            return None
        return [self.allocate() for _ in range(n)]

    def share(self, block: int) -> None:
        if self.ref[block] <= 0:
            raise ValueError(f"block {block} is not in use")
        self.ref[block] += 1

    def release(self, block: int) -> None:
        """Drop one reference; the last one returns the block to the free list.
        Its device contents are left as they are."""
        if self.ref[block] <= 0:
            raise ValueError(f"block {block} is not in use")
        self.ref[block] -= 1
        if self.ref[block] == 0:
            self._free.append(block)


def slots_of_positions(table: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Slot of each token position of one sequence: its block's first slot plus the
    offset inside the block."""
    table = np.asarray(table, np.int64)
    positions = np.asarray(positions, np.int64)
    return (table[positions // block_size] * block_size + positions % block_size).astype(np.int32)


def _cumsum0(lengths) -> np.ndarray:
    total = np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))])
    if total[-1] >= 2**31:
        raise ValueError("packed length exceeds int32")
    return total.astype(np.int32)


def _pad_tables(tables, width, pad):
    m = np.full((len(tables), width), pad, np.int32)
    for r, t in enumerate(tables):
        m[r, :len(t)] = t
    return m


@dataclass
class StepPlan:
    tables: list                        # per sequence, int32 block ids
    history_seq: np.ndarray             # per written-before-the-step token: sequence index
    history_pos: np.ndarray             # ... its position
    history_slots: np.ndarray           # ... its slot
    step_seq: np.ndarray                # the step's new tokens, same three arrays
    step_pos: np.ndarray
    step_slots: np.ndarray
    prefill: list                       # indices of prefill sequences
    decode: list                        # indices of decode sequences
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    max_seqlen_q: int
    max_seqlen_k: int
    prefill_block_tables: np.ndarray    # [len(prefill), width]
    context_lens: np.ndarray
    max_context_len: int
    decode_block_tables: np.ndarray     # [len(decode), width]
    table_width: int
    extra: dict = field(default_factory=dict)


def plan_step(seqs, block_size: int, pool: BlockPool, table_pad: int = -1) -> StepPlan:
    """Allocate blocks for every sequence (in order) and build the step's metadata.

    ``seqs`` are objects with ``phase``, ``context_len``, ``new_tokens``,
    ``prefix_group`` and ``prefix_len`` (workloads.SeqSpec).  A sequence whose
    prefix group was already seen reuses that sequence's prefix blocks with one
    more reference each; its prefix tokens are not written again.  Raises
    MemoryError if the pool runs out (the caller would preempt)."""
    bs = block_size
    tables, owner = [], {}
    for i, s in enumerate(seqs):
        n = -(-s.context_len // bs)
        shared = []
        if s.prefix_group >= 0:
            if s.prefix_len % bs:
                raise ValueError("a shared prefix must be a whole number of blocks")
            if s.prefix_group in owner:
                shared = list(tables[owner[s.prefix_group]][:s.prefix_len // bs])
                for b in shared:
                    pool.share(b)
            else:
                owner[s.prefix_group] = i
        own = pool.allocate_many(n - len(shared))
        if own is None:
            raise MemoryError(f"KV pool exhausted at sequence {i}")
        tables.append(np.array(shared + own, np.int32))

    hs, hp, ss, sp = [], [], [], []
    for i, s in enumerate(seqs):
        reuse = s.prefix_group >= 0 and owner[s.prefix_group] != i
        first = s.prefix_len if reuse else 0
        hp.append(np.arange(first, s.context_len - s.new_tokens, dtype=np.int64))
        hs.append(np.full(len(hp[-1]), i, np.int32))
        sp.append(np.arange(s.context_len - s.new_tokens, s.context_len, dtype=np.int64))
        ss.append(np.full(len(sp[-1]), i, np.int32))

    def slots(seq_idx, pos_list):
        parts = [slots_of_positions(tables[i], p, bs) for i, p in enumerate(pos_list)]
        return np.concatenate(parts) if parts else np.zeros(0, np.int32)

    prefill = [i for i, s in enumerate(seqs) if s.phase == "prefill"]
    decode = [i for i, s in enumerate(seqs) if s.phase == "decode"]
    width = max([len(t) for t in tables] + [1])
    lq = [seqs[i].new_tokens for i in prefill]
    lk = [seqs[i].context_len for i in prefill]
    ctx = np.array([seqs[i].context_len for i in decode], np.int32)
    return StepPlan(
        tables=tables,
        history_seq=np.concatenate(hs) if hs else np.zeros(0, np.int32),
        history_pos=np.concatenate(hp) if hp else np.zeros(0, np.int64),
        history_slots=slots(None, hp),
        step_seq=np.concatenate(ss) if ss else np.zeros(0, np.int32),
        step_pos=np.concatenate(sp) if sp else np.zeros(0, np.int64),
        step_slots=slots(None, sp),
        prefill=prefill, decode=decode,
        cu_seqlens_q=_cumsum0(lq), cu_seqlens_k=_cumsum0(lk),
        max_seqlen_q=max(lq, default=0), max_seqlen_k=max(lk, default=0),
        prefill_block_tables=_pad_tables([tables[i] for i in prefill], width, table_pad),
        context_lens=ctx, max_context_len=int(ctx.max()) if len(ctx) else 0,
        decode_block_tables=_pad_tables([tables[i] for i in decode], width, table_pad),
        table_width=width,
    )
