"""Paged KV-cache attention for AMD MI355X (gfx950): Python binding of libpkv.

Three calls, the data plane of a nano-vLLM-style engine (“Nano-vLLM 引擎架构解析” section 3.2 "PagedAttention"; “深入 Nano-vLLM 推理引擎” headings
"From Sequences to Blocks", "Control plane vs. data plane", "Prefill and
Decode", "Preparing for computation"):

* ``store_kvcache``  - write new tokens' K/V into their slots;
* ``paged_prefill``  - varlen causal attention over packed sequences, K/V read
  from the cache through block tables (cached prefix blocks included);
* ``paged_decode``   - one query per sequence over its cached context, streamed
  by wavefront workers over chunks of several kv heads' rows and merged where a
  context is cut.

This module only marshals arguments: shapes, dtypes and devices are checked,
pointers and torch's current stream are handed to the C ABI, and every step of
the computation runs in the HIP kernels.  There is no fallback: if libpkv.so is
not built, the first call raises.

Cache tensors are ``[num_blocks, block_size, num_kv_heads, head_dim]``
(float32 or bfloat16); metadata tensors are int32 on the same device.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import PkvError

__all__ = ["store_kvcache", "paged_prefill", "paged_decode", "paged_decode_workspace_size",
           "mixed_attention", "rotary_table", "PkvError", "version", "library_path", "timing_enable",
           "timing_collect", "timing_samples", "validate_store", "validate_prefill", "validate_decode",
           "contract_names", "debug_enable", "debug_enabled", "paged_decode_noalloc",
           "paged_decode_append"]

_DTYPES = {torch.float32: _lib.PKV_F32, torch.bfloat16: _lib.PKV_BF16}


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> int:
    return _lib.load().pkv_version()


def timing_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events on its stream (off by default)."""
    _lib.check(_lib.load().pkv_timing_enable(1 if on else 0))


def timing_collect() -> dict:
    """{kernel name: {launches, total_ms, avg_ms, min_ms, max_ms}} since the last collect."""
    lib = _lib.load()
    buf = (_lib.PkvKernelTiming * 32)()
    n = lib.pkv_timing_collect(buf, 32)
    if n < 0:
        _lib.check(n)
    out = {}
    for e in buf[:min(n, 32)]:
        out[e.kernel.decode()] = {"launches": e.launches, "total_ms": e.total_ms,
                                  "avg_ms": e.total_ms / max(e.launches, 1),
                                  "min_ms": e.min_ms, "max_ms": e.max_ms}
    return out


def timing_samples(capacity: int = 4096) -> list:
    """[(kernel name, ms)] of every launch recorded since the last collect, in launch
    order (consumes them, as timing_collect does)."""
    lib = _lib.load()
    buf = (_lib.PkvKernelSample * capacity)()
    n = lib.pkv_timing_samples(buf, capacity)
    if n < 0:
        _lib.check(n)
    return [(e.kernel.decode(), e.ms) for e in buf[:min(n, capacity)]]


def _cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor) -> _lib.PkvCache:
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_blocks, block_size, Hkv, D]")
    if k_cache.dtype not in _DTYPES or v_cache.dtype != k_cache.dtype:
        raise ValueError(f"cache dtype {k_cache.dtype} (float32 or bfloat16, both alike)")
    for t in (k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("caches must be contiguous device tensors")
    nb, bs, hkv, d = k_cache.shape
    return _lib.PkvCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, hkv, d,
                         _DTYPES[k_cache.dtype])


def _dev(t: torch.Tensor, name: str, dtype, like: torch.Tensor) -> int:
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != like.device or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous on {like.device}")
    return t.data_ptr()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def rotary_table(max_position: int, head_dim: int, base: float = 10000.0,
                 device="cuda") -> torch.Tensor:
    """The rotary table the ``rotary=`` arguments take: fp32 [max_position, head_dim],
    row p = cos(p * theta_i) for i < head_dim/2, then sin(p * theta_i), with
    theta_i = base^(-2i/head_dim) (RoFormer's frequencies), computed in float64."""
    i = torch.arange(head_dim // 2, dtype=torch.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = torch.arange(max_position, dtype=torch.float64)[:, None] * theta[None, :]
    return torch.cat([ang.cos(), ang.sin()], dim=1).to(torch.float32).to(device).contiguous()


def _rotary(rotary: torch.Tensor | None, like: torch.Tensor):
    if rotary is None:
        return None
    if rotary.dtype != torch.float32 or rotary.dim() != 2 or rotary.shape[1] != like.shape[3]:
        raise ValueError("rotary must be the fp32 [max_position, head_dim] table")
    _dev(rotary, "rotary", torch.float32, like)
    return _lib.PkvRotary(rotary.data_ptr(), rotary.shape[0])


def store_kvcache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                  positions: torch.Tensor | None = None,
                  rotary: torch.Tensor | None = None) -> None:
    """k, v [N, Hkv, D] -> rows slot_mapping[t] of the caches (slot -1 skipped).  With
    ``rotary`` (rotary_table) K is rotated at ``positions`` [N] int32 on the way in."""
    lib = _lib.load()
    desc = _cache_desc(k_cache, v_cache)
    n = slot_mapping.numel()
    if k.shape != (n,) + tuple(k_cache.shape[2:]) or v.shape != k.shape:
        raise ValueError(f"k, v must be [{n}, Hkv, D] like the cache rows")
    args = (_dev(k, "k", k_cache.dtype, k_cache), _dev(v, "v", k_cache.dtype, k_cache),
            _dev(slot_mapping, "slot_mapping", torch.int32, k_cache))
    rot = _rotary(rotary, k_cache)
    if rot is None:
        _lib.check(lib.pkv_store_kvcache(ctypes.byref(desc), *args, n, _stream(k_cache.device)))
        return
    if positions is None or positions.numel() != n:
        raise ValueError("rotary needs positions [N] int32")
    _lib.check(lib.pkv_store_kvcache_rotary(ctypes.byref(desc), *args,
                                            _dev(positions, "positions", torch.int32, k_cache),
                                            n, ctypes.byref(rot), _stream(k_cache.device)))


def paged_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                  block_tables: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                  scale: float, out: torch.Tensor | None = None,
                  rotary: torch.Tensor | None = None) -> torch.Tensor:
    """q [total_q, Hq, D] -> out [total_q, Hq, D]; sequences packed by cu_seqlens.  With
    ``rotary`` every query row is rotated at its position first."""
    lib = _lib.load()
    desc = _cache_desc(k_cache, v_cache)
    if q.dim() != 3 or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q must be [total_q, Hq, D]")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [batch, stride]")
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != batch + 1 or block_tables.shape[0] != batch:
        raise ValueError("cu_seqlens_q, cu_seqlens_k and block_tables disagree on batch")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    args = (_dev(q, "q", k_cache.dtype, k_cache), _dev(out, "out", k_cache.dtype, k_cache),
            q.shape[1], batch, _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, k_cache),
            _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, k_cache), int(max_seqlen_q),
            int(max_seqlen_k), _dev(block_tables, "block_tables", torch.int32, k_cache),
            block_tables.shape[1], float(scale))
    rot = _rotary(rotary, k_cache)
    if rot is None:
        _lib.check(lib.pkv_paged_prefill(ctypes.byref(desc), *args, _stream(k_cache.device)))
    else:
        _lib.check(lib.pkv_paged_prefill_rotary(ctypes.byref(desc), *args, ctypes.byref(rot),
                                                _stream(k_cache.device)))
    return out


def paged_decode_workspace_size(k_cache: torch.Tensor, v_cache: torch.Tensor, num_q_heads: int,
                                batch: int, max_context_len: int, num_workers: int = 0) -> int:
    desc = _cache_desc(k_cache, v_cache)
    return int(_lib.load().pkv_paged_decode_workspace_size(
        ctypes.byref(desc), num_q_heads, batch, max_context_len, num_workers))


def paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                 scale: float, num_workers: int = 0, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None,
                 rotary: torch.Tensor | None = None) -> torch.Tensor:
    """q [B, Hq, D] -> out [B, Hq, D]; one query per sequence over its context.  With
    ``rotary`` each query is rotated at position context_len - 1 first."""
    lib = _lib.load()
    desc = _cache_desc(k_cache, v_cache)
    if q.dim() != 3 or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q must be [B, Hq, D]")
    batch = q.shape[0]
    if context_lens.numel() != batch or block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise ValueError("context_lens / block_tables disagree with q on batch")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = lib.pkv_paged_decode_workspace_size(ctypes.byref(desc), q.shape[1], batch,
                                               int(max_context_len), int(num_workers))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_dev(q, "q", k_cache.dtype, k_cache), _dev(out, "out", k_cache.dtype, k_cache),
            q.shape[1], batch, _dev(context_lens, "context_lens", torch.int32, k_cache),
            int(max_context_len), _dev(block_tables, "block_tables", torch.int32, k_cache),
            block_tables.shape[1], float(scale), ws_ptr, ws_bytes, int(num_workers))
    rot = _rotary(rotary, k_cache)
    if rot is None:
        _lib.check(lib.pkv_paged_decode(ctypes.byref(desc), *args, _stream(k_cache.device)))
    else:
        _lib.check(lib.pkv_paged_decode_rotary(ctypes.byref(desc), *args, ctypes.byref(rot),
                                               _stream(k_cache.device)))
    return out


def paged_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor,
                        max_context_len: int, scale: float, num_workers: int = 0,
                        out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one call: k_new, v_new [B, Hkv, D] (each sequence's new token)
    go into the caches at slot_mapping [B] (the slot of position context_len - 1), and
    q [B, Hq, D] attends over the contexts that end with them.  Same bits as
    store_kvcache followed by paged_decode; one kernel (and the split merge) for bf16
    caches with one q head per kv head and blocks of at least one decode chunk, the
    two calls in turn otherwise."""
    lib = _lib.load()
    desc = _cache_desc(k_cache, v_cache)
    if q.dim() != 3 or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q must be [B, Hq, D]")
    batch = q.shape[0]
    if context_lens.numel() != batch or block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise ValueError("context_lens / block_tables disagree with q on batch")
    if k_new.shape != (batch,) + tuple(k_cache.shape[2:]) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new, v_new must be [{batch}, Hkv, D] like the cache rows")
    if slot_mapping.numel() != batch:
        raise ValueError("slot_mapping must hold one slot per sequence")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = lib.pkv_paged_decode_workspace_size(ctypes.byref(desc), q.shape[1], batch,
                                               int(max_context_len), int(num_workers))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(lib.pkv_paged_decode_append(
        ctypes.byref(desc), _dev(q, "q", k_cache.dtype, k_cache),
        _dev(k_new, "k_new", k_cache.dtype, k_cache), _dev(v_new, "v_new", k_cache.dtype, k_cache),
        _dev(out, "out", k_cache.dtype, k_cache), q.shape[1], batch,
        _dev(slot_mapping, "slot_mapping", torch.int32, k_cache),
        _dev(context_lens, "context_lens", torch.int32, k_cache), int(max_context_len),
        _dev(block_tables, "block_tables", torch.int32, k_cache), block_tables.shape[1],
        float(scale), ws_ptr, ws_bytes, int(num_workers), _stream(k_cache.device)))
    return out


def paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor,
                         max_context_len: int, scale: float, out: torch.Tensor,
                         num_workers: int = 0, rotary: torch.Tensor | None = None) -> torch.Tensor:
    """paged_decode through the entry point that allocates nothing: its split-K
    workspace is the library's fixed per-device array, and the caller passes ``out``."""
    lib = _lib.load()
    desc = _cache_desc(k_cache, v_cache)
    if q.dim() != 3 or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q must be [B, Hq, D]")
    batch = q.shape[0]
    if context_lens.numel() != batch or block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise ValueError("context_lens / block_tables disagree with q on batch")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    rot = _rotary(rotary, k_cache)
    _lib.check(lib.pkv_paged_decode_noalloc(
        ctypes.byref(desc), _dev(q, "q", k_cache.dtype, k_cache),
        _dev(out, "out", k_cache.dtype, k_cache), q.shape[1], batch,
        _dev(context_lens, "context_lens", torch.int32, k_cache), int(max_context_len),
        _dev(block_tables, "block_tables", torch.int32, k_cache), block_tables.shape[1],
        float(scale), int(num_workers), None if rot is None else ctypes.byref(rot),
        _stream(k_cache.device)))
    return out


def mixed_attention(k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float,
                    q_prefill: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, prefill_tables: torch.Tensor, max_seqlen_q: int,
                    max_seqlen_k: int, q_decode: torch.Tensor, decode_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_context_len: int, num_workers: int = 0,
                    out_prefill: torch.Tensor | None = None,
                    out_decode: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None,
                    rotary: torch.Tensor | None = None):
    """Prefill of some sequences and decode of others in one call (one kernel launch for
    the common bf16 shapes); returns (out_prefill, out_decode), bit-identical to
    paged_prefill and paged_decode called one after the other."""
    lib = _lib.load()
    desc = _cache_desc(k_cache, v_cache)
    hq = q_decode.shape[1] if q_decode.numel() else q_prefill.shape[1]
    pb = cu_seqlens_q.numel() - 1
    db = q_decode.shape[0]
    if out_prefill is None:
        out_prefill = torch.empty_like(q_prefill)
    if out_decode is None:
        out_decode = torch.empty_like(q_decode)
    need = lib.pkv_paged_decode_workspace_size(ctypes.byref(desc), hq, max(db, 1),
                                               int(max(max_context_len, 1)), int(num_workers))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_cache.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptr = lambda t, name, dt: _dev(t, name, dt, k_cache) if t.numel() else None
    rot = _rotary(rotary, k_cache)
    _lib.check(lib.pkv_mixed_attention(
        ctypes.byref(desc), hq, float(scale),
        ptr(q_prefill, "q_prefill", k_cache.dtype), ptr(out_prefill, "out_prefill", k_cache.dtype),
        pb, _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, k_cache),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, k_cache), int(max_seqlen_q),
        int(max_seqlen_k), ptr(prefill_tables, "prefill_tables", torch.int32),
        prefill_tables.shape[1] if prefill_tables.dim() == 2 else 0,
        ptr(q_decode, "q_decode", k_cache.dtype), ptr(out_decode, "out_decode", k_cache.dtype),
        db, ptr(context_lens, "context_lens", torch.int32), int(max_context_len),
        ptr(decode_tables, "decode_tables", torch.int32),
        decode_tables.shape[1] if decode_tables.dim() == 2 else 0, ws_ptr, ws_bytes,
        int(num_workers), None if rot is None else ctypes.byref(rot), _stream(k_cache.device)))
    return out_prefill, out_decode


# ---- contract checks of the metadata arrays (the library's pkv_validate_*) ----

def _meta(a, name: str):
    """(pointer, on_host, keepalive) of an int32 metadata array: a numpy array or CPU
    tensor is checked on the host, a device tensor on its device."""
    import numpy as np
    if isinstance(a, torch.Tensor):
        if a.dtype != torch.int32:
            raise ValueError(f"{name} must be int32, got {a.dtype}")
        a = a.contiguous()
        return a.data_ptr(), (not a.is_cuda), a
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr.ctypes.data, True, arr


def _meta_desc(num_blocks: int, block_size: int) -> _lib.PkvCache:
    return _lib.PkvCache(None, None, int(num_blocks), int(block_size), 1, 128, _lib.PKV_BF16)


def _run_check(fn, device_arrays, *args) -> int:
    bits = ctypes.c_uint32(0)
    stream = None
    for t in device_arrays:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            stream = _stream(t.device)
    st = fn(*args, ctypes.byref(bits), stream)
    if st not in (_lib.PKV_OK, _lib.PKV_ERR_INVALID) or (st == _lib.PKV_ERR_INVALID and
                                                         bits.value == 0):
        _lib.check(st)
    return int(bits.value)


def validate_store(slot_mapping, num_blocks: int, block_size: int) -> int:
    """Contract bits (0 = every contract holds) of a KV write's slot mapping: slots in
    [0, num_blocks*block_size) or -1, no valid slot twice."""
    lib = _lib.load()
    ptr, host, keep = _meta(slot_mapping, "slot_mapping")
    n = keep.numel() if isinstance(keep, torch.Tensor) else keep.size
    return _run_check(lib.pkv_validate_store, [slot_mapping],
                      ctypes.byref(_meta_desc(num_blocks, block_size)), ptr, n, int(host))


def validate_prefill(cu_seqlens_q, cu_seqlens_k, block_tables, max_seqlen_q: int,
                     max_seqlen_k: int, num_blocks: int, block_size: int) -> int:
    """Contract bits of a prefill's cumulative lengths and block tables."""
    lib = _lib.load()
    pq, hq, kq = _meta(cu_seqlens_q, "cu_seqlens_q")
    pk, hk, kk = _meta(cu_seqlens_k, "cu_seqlens_k")
    pt, ht, kt = _meta(block_tables, "block_tables")
    if not (hq == hk == ht):
        raise ValueError("metadata arrays must all be on the host or all on the device")
    batch = (kq.numel() if isinstance(kq, torch.Tensor) else kq.size) - 1
    stride = kt.shape[1] if kt.ndim == 2 else 0
    if kt.shape[0] != batch or (kk.numel() if isinstance(kk, torch.Tensor) else kk.size) != batch + 1:
        raise ValueError("cu_seqlens_q, cu_seqlens_k and block_tables disagree on batch")
    return _run_check(lib.pkv_validate_prefill, [cu_seqlens_q],
                      ctypes.byref(_meta_desc(num_blocks, block_size)), batch, pq, pk,
                      int(max_seqlen_q), int(max_seqlen_k), pt, stride, int(hq))


def validate_decode(context_lens, block_tables, max_context_len: int, num_blocks: int,
                    block_size: int) -> int:
    """Contract bits of a decode's context lengths and block tables."""
    lib = _lib.load()
    pc, hc, kc = _meta(context_lens, "context_lens")
    pt, ht, kt = _meta(block_tables, "block_tables")
    if hc != ht:
        raise ValueError("metadata arrays must all be on the host or all on the device")
    batch = kc.numel() if isinstance(kc, torch.Tensor) else kc.size
    stride = kt.shape[1] if kt.ndim == 2 else 0
    if kt.shape[0] != batch:
        raise ValueError("context_lens and block_tables disagree on batch")
    return _run_check(lib.pkv_validate_decode, [context_lens],
                      ctypes.byref(_meta_desc(num_blocks, block_size)), batch, pc,
                      int(max_context_len), pt, stride, int(hc))


def contract_names(bits: int) -> list:
    """The violated contracts a validate_* result names."""
    return [v for k, v in _lib.CONTRACTS.items() if bits & k]


def debug_enable(on: bool = True) -> None:
    """Debug mode: every data-plane call checks its device metadata first and fails with
    PkvError instead of launching (initially on when PKV_DEBUG is set and not "0")."""
    _lib.check(_lib.load().pkv_debug_enable(1 if on else 0))


def debug_enabled() -> bool:
    return bool(_lib.load().pkv_debug_enabled())
