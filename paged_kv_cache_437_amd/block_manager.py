"""Python view of the C++ block manager (``pkv_bm_*`` in include/pkv.h).

The host control plane that hands out KV block ids: a fixed pool whose free deque is
handed out from its head, reference counts, and a prefix cache that maps the hash of
every full block (chained over the blocks before it) to the block holding it, so a
new sequence whose leading blocks are cached takes those blocks with one more
reference instead of recomputing them (“Nano-vLLM 引擎架构解析” section 3.2
"PagedAttention"; “深入 Nano-vLLM 推理引擎”, "From Sequences to Blocks", "Prefix Caching by
hashing", "Control plane vs. data plane", "Handling resource exhaustion").  Argument
marshalling only: every rule runs in the library.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

__all__ = ["BlockManager", "PoolExhausted"]


class PoolExhausted(_lib.PkvError):
    """Too few free blocks: the scheduler preempts a sequence and tries again."""


def _check(status: int) -> int:
    if status == _lib.PKV_ERR_NO_BLOCKS:
        raise PoolExhausted(status, _lib.load().pkv_last_error().decode())
    if status < 0:
        _lib.check(status)
    return status


class BlockManager:
    """One pool of ``num_blocks`` blocks of ``block_size`` tokens."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        lib = _lib.load()
        self._lib = lib
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.shape != (self.num_blocks,):
                raise ValueError("free_order must hold num_blocks ids")
        handle = ctypes.c_void_p()
        _check(lib.pkv_bm_create(self.num_blocks, self.block_size,
                                 None if order is None else order.ctypes.data,
                                 ctypes.byref(handle)))
        self._h = handle

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return _check(self._lib.pkv_bm_num_free(self._h))

    def ref_count(self, block: int) -> int:
        return _check(self._lib.pkv_bm_ref_count(self._h, int(block)))

    def add_sequence(self, token_ids) -> int:
        toks = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32))
        seq = ctypes.c_int64()
        _check(self._lib.pkv_bm_add_sequence(self._h, toks.ctypes.data, int(toks.size),
                                             ctypes.byref(seq)))
        return seq.value

    def remove_sequence(self, seq: int) -> None:
        _check(self._lib.pkv_bm_remove_sequence(self._h, int(seq)))

    def can_allocate(self, seq: int) -> bool:
        return _check(self._lib.pkv_bm_can_allocate(self._h, int(seq))) == 1

    def allocate(self, seq: int) -> None:
        """Blocks for all of the sequence's tokens; raises PoolExhausted (nothing taken)."""
        _check(self._lib.pkv_bm_allocate(self._h, int(seq)))

    def num_cached_tokens(self, seq: int) -> int:
        return _check(self._lib.pkv_bm_num_cached_tokens(self._h, int(seq)))

    def num_tokens(self, seq: int) -> int:
        return _check(self._lib.pkv_bm_num_tokens(self._h, int(seq)))

    def can_append(self, seq: int) -> bool:
        return _check(self._lib.pkv_bm_can_append(self._h, int(seq))) == 1

    def append_token(self, seq: int, token_id: int) -> None:
        _check(self._lib.pkv_bm_append_token(self._h, int(seq), int(token_id)))

    def deallocate(self, seq: int) -> None:
        _check(self._lib.pkv_bm_deallocate(self._h, int(seq)))

    def block_table(self, seq: int) -> np.ndarray:
        n = _check(self._lib.pkv_bm_block_table(self._h, int(seq), None, 0))
        out = np.zeros(n, np.int32)
        if n:
            _check(self._lib.pkv_bm_block_table(self._h, int(seq), out.ctypes.data, n))
        return out
