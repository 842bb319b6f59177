"""Rotary position embedding, plain (test infrastructure only).

“基于 nano-vLLM 学习大模型推理关键功能” section 3.3 lists rotary_embedding among the layers a
model is built from; the pages give no formula.  The formula is RoFormer's (Su et
al., 2021, "RoFormer: Enhanced Transformer with Rotary Position Embedding"): the
head dimension is split into pairs, each rotated by the angle position * theta_i with
theta_i = base^(-2i/D).  Reading: the half-split pairing (element i with element
i + D/2), base 10000 unless a caller says otherwise.  Everything float64.

``rotate`` is the definition; ``round_to_bf16`` rounds float64 values to bfloat16 by
the definition of round-to-nearest-even (no detour through float32, which would
round twice); ``rotary_step`` is a workload with K rotated at every token's position
and stored in the cache's element type, and each query rotated at its own position
(query i of Lq new tokens over Lk keys sits at Lk - Lq + i), ready for ``run_step``.
"""
from __future__ import annotations

import copy

import numpy as np

from .paged_attention import as_float

__all__ = ["rotate", "round_to_bf16", "rotary_step"]


def rotate(x, positions, base: float = 10000.0) -> np.ndarray:
    """x [..., n, H, D] (or [n, D]) rotated at positions [n]: pair (i, i + D/2) by the
    angle positions * base^(-2i/D)."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    h = D // 2
    theta = base ** (-2.0 * np.arange(h, dtype=np.float64) / D)
    ang = np.asarray(positions, np.float64)[:, None] * theta[None, :]  # [n, h]
    c, s = np.cos(ang), np.sin(ang)
    if x.ndim >= 3:  # [..., n, H, D]: broadcast over heads
        c, s = c[:, None, :], s[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), round to nearest, ties to even: the
    significand is kept to 8 bits (frexp gives it in [0.5, 1)) with numpy's
    half-to-even rint.  Finite normal inputs only."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0) / 256.0, e)  # exactly representable in float32
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _store_type(values, dtype: str):
    return round_to_bf16(values) if dtype == "bf16" else values.astype(np.float32)


def rotary_step(wl, base: float = 10000.0):
    """A copy of the workload whose K are rotated at each token's position (in the
    cache's element type) and whose queries are rotated at their positions (float64)."""
    out = copy.copy(wl)
    out.k = [_store_type(rotate(as_float(k), np.arange(len(k)), base), wl.dtype) for k in wl.k]
    qs = []
    for i, q in enumerate(wl.q):
        s = wl.seqs[i]
        pos = np.arange(s.context_len - s.new_tokens, s.context_len)
        qs.append(rotate(as_float(q), pos, base) if len(q) else as_float(q))
    out.q = qs
    return out
