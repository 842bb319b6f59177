"""One whole step of a workload on the CPU (test infrastructure only).

The step follows the pages' order for a batch: blocks are allocated by the
control plane, the new tokens' K/V are written into their slots, then prefill
runs over the prefill sequences and decode over the decode sequences (“深入 Nano-vLLM 推理引擎”,
headings "Prefill and Decode" and "Preparing for computation").  Tokens
a sequence already had before the step (decode history, a cached prefix) are
written by an earlier KV write.  Every slot that no token writes keeps the
``stale`` value, standing for whatever a freed block held before ("Control plane
vs. data plane": freed blocks are not cleared).
"""
from __future__ import annotations

import numpy as np

from .block_manager import plan_step
from .paged_attention import paged_decode, paged_prefill, store_kvcache

__all__ = ["stale_value", "build_caches", "run_step"]

# a quiet NaN in each storage format
_STALE = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0)}


def stale_value(dtype: str):
    return _STALE[dtype]


def _rows(wl, triples):
    """K rows, V rows and slots of the listed (seq, position, slot) triples, in order."""
    raw = np.float32 if wl.dtype == "f32" else np.uint16
    shape = (len(triples), wl.num_kv_heads, wl.head_dim)
    k = np.empty(shape, raw)
    v = np.empty(shape, raw)
    for n, (i, p, _) in enumerate(triples):
        k[n] = wl.k[i][p]
        v[n] = wl.v[i][p]
    return k, v, [s for (_, _, s) in triples]


def build_caches(wl, plan, stale=None):
    """Pool arrays after the history write and the step's KV write."""
    raw = np.float32 if wl.dtype == "f32" else np.uint16
    fill = stale_value(wl.dtype) if stale is None else stale
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
    k_cache = np.full(shape, fill, raw)
    v_cache = np.full(shape, fill, raw)
    for part in ("history_slots", "step_slots"):
        k, v, slots = _rows(wl, plan[part])
        store_kvcache(k_cache, v_cache, k, v, slots)
    return k_cache, v_cache


def run_step(wl, plan=None, stale=None, dtype=np.float64) -> dict:
    """Outputs of the step: prefill rows [sum Lq, Hq, D] and decode rows [B, Hq, D]."""
    plan = plan_step(wl) if plan is None else plan
    k_cache, v_cache = build_caches(wl, plan, stale)
    out = {"plan": plan, "k_cache": k_cache, "v_cache": v_cache}
    pre = plan["prefill"]
    if pre:
        q = np.concatenate([wl.q[i] for i in pre])
        out["prefill"] = paged_prefill(q, k_cache, v_cache, plan["cu_seqlens_q"],
                                       plan["cu_seqlens_k"], plan["prefill_block_tables"],
                                       wl.scale, dtype)
    dec = plan["decode"]
    if dec:
        q = np.stack([wl.q[i][0] for i in dec])
        out["decode"] = paged_decode(q, k_cache, v_cache, plan["decode_block_tables"],
                                     plan["context_lens"], wl.scale, dtype)
    return out
