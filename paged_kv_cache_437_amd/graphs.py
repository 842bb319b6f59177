"""A decode step captured once in a HIP graph and replayed.

“深入 Nano-vLLM 推理引擎”, "CUDA Graphs": a decode step is short enough that launching its
kernels one by one costs a noticeable share of it, so the engine records the
step's GPU work once per common batch size and replays it.  ``DecodeStepGraph``
does that for the hot path of a decode step: the KV write of one new token per
sequence (``store_kvcache``) and ``paged_decode`` (its streaming and merge
kernels), captured with torch's graph API on static device buffers.  ``run``
copies a batch into the static buffers and replays; a batch smaller than the
captured size is padded with rows that write nothing (slot -1, “Nano-vLLM”'s padding
convention) and read one token of a valid block, and their outputs are dropped.

Argument marshalling only: the captured work is the library's kernels, and the
graph records no memset (the library issues none).
"""
from __future__ import annotations

import torch

from . import paged_decode, paged_decode_workspace_size, store_kvcache

__all__ = ["DecodeStepGraph"]


class DecodeStepGraph:
    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, num_q_heads: int,
                 batch: int, table_width: int, scale: float, num_workers: int = 0):
        if batch < 1 or table_width < 1:
            raise ValueError("batch and table_width must be >= 1")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.batch, self.width, self.scale = int(batch), int(table_width), float(scale)
        self.num_workers = int(num_workers)
        nb, bs, hkv, d = k_cache.shape
        self.max_context_len = self.width * bs
        dev, dt = k_cache.device, k_cache.dtype
        self.q = torch.zeros((batch, num_q_heads, d), dtype=dt, device=dev)
        self.k_new = torch.zeros((batch, hkv, d), dtype=dt, device=dev)
        self.v_new = torch.zeros((batch, hkv, d), dtype=dt, device=dev)
        self.slots = torch.full((batch,), -1, dtype=torch.int32, device=dev)
        self.tables = torch.zeros((batch, self.width), dtype=torch.int32, device=dev)
        self.context_lens = torch.ones((batch,), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        ws = paged_decode_workspace_size(k_cache, v_cache, num_q_heads, batch,
                                         self.max_context_len, self.num_workers)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)

        # the first calls (device queries, code loading) run outside the capture
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            self._step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step()

    def _step(self):
        store_kvcache(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots)
        paged_decode(self.q, self.k_cache, self.v_cache, self.tables, self.context_lens,
                     self.max_context_len, self.scale, num_workers=self.num_workers,
                     out=self.out, workspace=self.workspace)

    def run(self, q, k_new, v_new, slot_mapping, block_tables, context_lens) -> torch.Tensor:
        """One decode step for n <= batch sequences: q [n, Hq, D], k_new / v_new
        [n, Hkv, D], slot_mapping [n], block_tables [n, w <= table_width] and
        context_lens [n] (int32, device).  Returns out[:n] (a view of the static
        output: copy it before the next run)."""
        n = q.shape[0]
        if n > self.batch or block_tables.shape[1] > self.width:
            raise ValueError(f"batch {n} / table width {block_tables.shape[1]} exceed the "
                             f"captured {self.batch} / {self.width}")
        self.q[:n].copy_(q)
        self.k_new[:n].copy_(k_new)
        self.v_new[:n].copy_(v_new)
        self.slots[:n].copy_(slot_mapping)
        self.tables[:n, :block_tables.shape[1]].copy_(block_tables)
        self.tables[:n, block_tables.shape[1]:].fill_(0)
        self.context_lens[:n].copy_(context_lens)
        if n < self.batch:  # padding rows: write nothing, read token 0 of block 0
            self.slots[n:].fill_(-1)
            self.tables[n:].fill_(0)
            self.context_lens[n:].fill_(1)
        self.graph.replay()
        return self.out[:n]
