"""Plain CPU definition of paged KV-cache attention (test infrastructure only).

What is computed, and where the pages say so (“Nano-vLLM 引擎架构解析”,
section 3.2 "PagedAttention"; “深入 Nano-vLLM 推理引擎”,
headings "From Sequences to Blocks", "Prefix Caching by hashing",
"Control plane vs. data plane", "Preparing for computation", "Prefill and
Decode"):

* KV memory is a fixed pool of blocks; a sequence's tokens live in the blocks its
  block table lists, in order; a block holds ``block_size`` consecutive tokens.
* The KV write puts each new token's K and V into its slot; a freed block is not
  cleared and a later write simply overwrites it.
* Prefill runs once per sequence over its new tokens, packed by cumulative
  lengths; decode adds one token per sequence.  Both are ordinary softmax
  attention over the sequence's logical tokens; paging changes where the rows
  live, not what is computed.

Readings where the pages are silent (the pages leave the attention layer itself
to a second part that is not included):

* cache layout ``[num_blocks, block_size, num_kv_heads, head_dim]``; slot ``s``
  is block ``s // block_size``, offset ``s % block_size``; slot -1 is skipped;
* q head ``h`` reads kv head ``h // (Hq // Hkv)``;
* causal alignment is bottom-right: with ``Lq`` queries over ``Lk`` keys, query
  ``i`` sits at position ``Lk - Lq + i`` and sees keys ``0 .. Lk - Lq + i``;
* decode is prefill with one query over ``context_len`` keys (the new token's
  K/V is written first and is the last key);
* split-K: a decode context is cut at block boundaries into ranges, each range
  gives (m, l, o) = (max score, sum of exp(score - m), sum of exp(score - m) v),
  and the ranges merge as out = sum_i e^(m_i - M) o_i / sum_i e^(m_i - M) l_i
  with M = max_i m_i.

All floating-point arithmetic is float64 unless a caller asks for float32.
Nothing here is tuned; every loop is over sequences and heads, one at a time.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_float", "as_float", "store_kvcache", "gather_tokens", "causal_attention",
    "paged_prefill", "paged_decode", "decode_split_partials", "combine_partials",
    "kv_head_of",
]


def bf16_bits_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32; widen exactly."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(dtype)


def store_kvcache(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
                  slot_mapping) -> None:
    """Write token t's K/V rows into slot ``slot_mapping[t]``, in place.

    Caches are ``[num_blocks, block_size, Hkv, D]`` of any element type (the copy
    is exact, element for element).  Slot -1 means "no write".  A slot outside
    the pool, or the same slot twice in one call, is an error.
    (KV write of the "Control plane vs. data plane" heading: reuse overwrites.)
    """
    num_blocks, block_size = k_cache.shape[0], k_cache.shape[1]
    written = set()
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot == -1:
            continue
        if slot < 0 or slot >= num_blocks * block_size:
            raise ValueError(f"slot {slot} of token {t} is outside the pool")
        if slot in written:
            raise ValueError(f"slot {slot} written twice in one call")
        written.add(slot)
        block, offset = divmod(slot, block_size)
        k_cache[block, offset] = k[t]
        v_cache[block, offset] = v[t]


def as_float(x: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Values as floats: uint16 arrays hold bf16 bit patterns, anything else is cast."""
    x = np.asarray(x)
    return bf16_bits_to_float(x, dtype) if x.dtype == np.uint16 else x.astype(dtype)


def gather_tokens(cache: np.ndarray, table_row, length: int) -> np.ndarray:
    """Logical token rows 0..length-1 of one sequence: token j is in block
    ``table_row[j // block_size]`` at offset ``j % block_size`` ("From Sequences
    to Blocks": a long sequence spans several blocks, in order)."""
    block_size = cache.shape[1]
    rows = [cache[int(table_row[j // block_size]), j % block_size] for j in range(length)]
    if not rows:
        return np.empty((0,) + cache.shape[2:], cache.dtype)
    return np.stack(rows)


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped heads: q heads are split into Hkv consecutive groups of Hq/Hkv."""
    return q_head // (num_q_heads // num_kv_heads)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     dtype=np.float64) -> np.ndarray:
    """softmax(scale * q k^T, bottom-right causal) v for one sequence.

    q [Lq, Hq, D]; k, v [Lk, Hkv, D]; returns [Lq, Hq, D] in ``dtype``.
    Query i sits at position Lk - Lq + i and sees keys 0 .. Lk - Lq + i.
    """
    Lq, Hq, D = q.shape
    Lk, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    if Lq > Lk or (Lq > 0 and Lk == 0):
        raise ValueError("need Lk >= Lq and at least one key")
    out = np.zeros((Lq, Hq, D), dtype)
    if Lq == 0:
        return out
    sees = np.arange(Lk)[None, :] <= (Lk - Lq + np.arange(Lq))[:, None]  # [Lq, Lk]
    for h in range(Hq):
        kh = kv_head_of(h, Hq, Hkv)
        qh = as_float(q[:, h, :], dtype)
        kk = as_float(k[:, kh, :], dtype)
        vv = as_float(v[:, kh, :], dtype)
        scores = (qh @ kk.T) * dtype(scale)
        scores = np.where(sees, scores, -np.inf)
        p = np.exp(scores - scores.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vv
    return out


def paged_prefill(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, scale,
                  dtype=np.float64) -> np.ndarray:
    """Packed varlen prefill ("Preparing for computation": prefill batches several
    sequences and computes cumulative sequence lengths).  Sequence b owns query
    rows cu_q[b]..cu_q[b+1]-1 and keys 0..Lk-1 with Lk = cu_k[b+1]-cu_k[b], read
    from the cache through block_tables[b] ("Prefix Caching": a cached prefix is
    read, not recomputed).  Arrays may be float or bf16 bit patterns (uint16)."""
    out = np.zeros(q.shape, dtype)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        Lk = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        if q1 == q0:
            continue
        K = gather_tokens(k_cache, block_tables[b], Lk)
        V = gather_tokens(v_cache, block_tables[b], Lk)
        out[q0:q1] = causal_attention(q[q0:q1], K, V, scale, dtype)
    return out


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                 dtype=np.float64) -> np.ndarray:
    """Decode ("Prefill and Decode": one new token per sequence per step): q
    [B, Hq, D], one query per sequence over its context_lens[b] cached tokens."""
    out = np.zeros(q.shape, dtype)
    for b in range(q.shape[0]):
        L = int(context_lens[b])
        K = gather_tokens(k_cache, block_tables[b], L)
        V = gather_tokens(v_cache, block_tables[b], L)
        out[b] = causal_attention(q[b:b + 1], K, V, scale, dtype)[0]
    return out


def decode_split_partials(q_row, k, v, scale, bounds, dtype=np.float64):
    """Per-range partials of one decode query.

    q_row [Hq, D]; k, v [L, Hkv, D]; ``bounds`` = [0, b1, ..., L] cut points.
    Returns m [S, Hq], l [S, Hq], o [S, Hq, D] with, for range i and head h,
    m = max score, l = sum exp(score - m), o = sum exp(score - m) * v.
    """
    Hq, D = np.shape(q_row)
    Hkv = k.shape[1]
    S = len(bounds) - 1
    m = np.full((S, Hq), -np.inf, dtype)
    l = np.zeros((S, Hq), dtype)
    o = np.zeros((S, Hq, D), dtype)
    for i in range(S):
        a, b = int(bounds[i]), int(bounds[i + 1])
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            s = (as_float(k[a:b, kh], dtype) @ as_float(q_row[h], dtype)) * dtype(scale)
            m[i, h] = s.max()
            e = np.exp(s - m[i, h])
            l[i, h] = e.sum()
            o[i, h] = e @ as_float(v[a:b, kh], dtype)
    return m, l, o


def combine_partials(m, l, o):
    """Merge split partials: M = max_i m_i; out = sum e^(m_i-M) o_i / sum e^(m_i-M) l_i."""
    M = m.max(axis=0)
    w = np.exp(m - M[None, :])  # [S, Hq]
    return (w[:, :, None] * o).sum(axis=0) / (w * l).sum(axis=0)[:, None]
