"""One step of the data plane on the device: KV write, then prefill and decode.

``DeviceStep`` takes a synthetic workload (shapes, pool, free-list order, values),
plans its blocks with the control plane, allocates the pool on the device,
writes every token the sequences already had before the step (decode history,
cached prefixes), and keeps all of the step's inputs resident in device memory.
``run()`` then enqueues exactly the hot path: ``store_kvcache`` of the step's new
tokens, ``paged_prefill`` over the prefill sequences and ``paged_decode`` over the
decode sequences, on torch's current stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (contract_names, mixed_attention, paged_decode, paged_decode_append,
               paged_decode_workspace_size,
               paged_prefill, store_kvcache, validate_decode, validate_prefill, validate_store)
from .control import BlockPool, plan_step

__all__ = ["DeviceStep", "check_plan", "to_device_values", "STALE_BITS"]


def check_plan(plan, num_blocks: int, block_size: int) -> None:
    """The data-plane contracts on the control plane's host copies of a step's metadata,
    before any of it reaches the device (the library's host-side checks): slots in the
    pool and written once per call, used table entries in the pool, consistent lengths,
    tables wide enough.  Raises ValueError naming what is violated."""
    checks = [("history KV write", validate_store(plan.history_slots, num_blocks, block_size)),
              ("step KV write", validate_store(plan.step_slots, num_blocks, block_size))]
    if plan.prefill:
        checks.append(("prefill", validate_prefill(
            plan.cu_seqlens_q, plan.cu_seqlens_k, plan.prefill_block_tables, plan.max_seqlen_q,
            plan.max_seqlen_k, num_blocks, block_size)))
    if plan.decode:
        checks.append(("decode", validate_decode(plan.context_lens, plan.decode_block_tables,
                                                 plan.max_context_len, num_blocks, block_size)))
    bad = [f"{what}: {'; '.join(contract_names(bits))}" for what, bits in checks if bits]
    if bad:
        raise ValueError("step metadata violates the data-plane contract: " + " | ".join(bad))

# bit patterns used to poison pool memory no token writes
STALE_BITS = {
    "nan": {"f32": 0x7FC00000, "bf16": 0x7FC0},
    "inf": {"f32": 0x7F800000, "bf16": 0x7F80},
    "-inf": {"f32": 0xFF800000, "bf16": 0xFF80},
    "huge": {"f32": 0x7149F2CA, "bf16": 0x7149},
}


def to_device_values(a: np.ndarray, device) -> torch.Tensor:
    """float32 array, or uint16 bf16 bit patterns, as a device tensor of that type."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def _fill_bits(t: torch.Tensor, bits: int) -> None:
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(bits - 0x10000 if bits >= 0x8000 else bits)
    else:
        t.view(torch.int32).fill_(bits - 0x100000000 if bits >= 0x80000000 else bits)


class DeviceStep:
    def __init__(self, wl, device="cuda", stale: str | None = "nan", table_pad: int = -1,
                 num_workers: int = 0, plan=None, rotary: torch.Tensor | None = None):
        """``rotary``: a rotary_table; K is then rotated at each token's position as it
        is written (history and step alike) and queries are rotated at theirs."""
        self.wl = wl
        self.device = torch.device(device)
        self.num_workers = num_workers
        self.rotary = rotary
        pool = BlockPool(wl.num_blocks, wl.free_order)
        self.plan = plan if plan is not None else plan_step(wl.seqs, wl.block_size, pool,
                                                            table_pad)
        p = self.plan
        check_plan(p, wl.num_blocks, wl.block_size)
        dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
        self.k_cache = torch.empty(shape, dtype=dt, device=self.device)
        self.v_cache = torch.empty(shape, dtype=dt, device=self.device)
        if stale is not None:
            _fill_bits(self.k_cache, STALE_BITS[stale][wl.dtype])
            _fill_bits(self.v_cache, STALE_BITS[stale][wl.dtype])

        def rows(seq_idx, pos):
            if len(seq_idx) == 0:
                e = np.zeros((0, wl.num_kv_heads, wl.head_dim),
                             np.float32 if wl.dtype == "f32" else np.uint16)
                return e, e
            ks, vs = [], []
            starts = np.flatnonzero(np.r_[True, seq_idx[1:] != seq_idx[:-1]])
            ends = np.r_[starts[1:], len(seq_idx)]
            for a, b in zip(starts, ends):
                i = int(seq_idx[a])
                ks.append(wl.k[i][pos[a]:pos[b - 1] + 1])
                vs.append(wl.v[i][pos[a]:pos[b - 1] + 1])
            return np.concatenate(ks), np.concatenate(vs)

        dev = self.device
        hk, hv = rows(p.history_seq, p.history_pos)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
        if len(p.history_slots):
            store_kvcache(to_device_values(hk, dev), to_device_values(hv, dev), self.k_cache,
                          self.v_cache, torch.from_numpy(p.history_slots).to(dev),
                          positions=i32(p.history_pos), rotary=rotary)
        del hk, hv
        sk, sv = rows(p.step_seq, p.step_pos)
        self.k_new = to_device_values(sk, dev)
        self.v_new = to_device_values(sv, dev)
        self.slot_mapping = torch.from_numpy(p.step_slots).to(dev)
        self.positions = i32(p.step_pos)

        self.q_prefill = self.q_decode = None
        self._append_rows = None
        if p.prefill:
            self.q_prefill = to_device_values(np.concatenate([wl.q[i] for i in p.prefill]), dev)
            self.cu_seqlens_q = i32(p.cu_seqlens_q)
            self.cu_seqlens_k = i32(p.cu_seqlens_k)
            self.prefill_tables = i32(p.prefill_block_tables)
            self.out_prefill = torch.empty_like(self.q_prefill)
        if p.decode:
            self.q_decode = to_device_values(np.stack([wl.q[i][0] for i in p.decode]), dev)
            self.context_lens = i32(p.context_lens)
            self.decode_tables = i32(p.decode_block_tables)
            self.out_decode = torch.empty_like(self.q_decode)
            ws = paged_decode_workspace_size(self.k_cache, self.v_cache, wl.num_q_heads,
                                             len(p.decode), p.max_context_len, num_workers)
            self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)

    # the three calls of the hot path, separately (for per-kernel timing) and together
    def store(self):
        store_kvcache(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slot_mapping,
                      positions=self.positions, rotary=self.rotary)

    def prefill(self):
        if self.q_prefill is None:
            return None
        p = self.plan
        return paged_prefill(self.q_prefill, self.k_cache, self.v_cache, self.cu_seqlens_q,
                             self.cu_seqlens_k, self.prefill_tables, p.max_seqlen_q,
                             p.max_seqlen_k, self.wl.scale, out=self.out_prefill,
                             rotary=self.rotary)

    def decode(self):
        if self.q_decode is None:
            return None
        p = self.plan
        return paged_decode(self.q_decode, self.k_cache, self.v_cache, self.decode_tables,
                            self.context_lens, p.max_context_len, self.wl.scale,
                            num_workers=self.num_workers, out=self.out_decode,
                            workspace=self.workspace, rotary=self.rotary)

    def run(self):
        self.store()
        self.prefill()
        self.decode()
        return self

    def decode_append(self):
        """A decode-only step in one call: the decode sequences' new tokens are written
        by the decode itself (paged_decode_append; same bits as store() + decode())."""
        if self.q_decode is None:
            return None
        if self.q_prefill is not None or self.rotary is not None:
            raise ValueError("decode_append covers decode-only steps without rotary")
        p = self.plan
        if self._append_rows is None:
            where = {int(s): t for t, s in enumerate(p.step_seq)}
            idx = torch.tensor([where[i] for i in p.decode], dtype=torch.long,
                               device=self.device)
            self._append_rows = (self.k_new.index_select(0, idx).contiguous(),
                                 self.v_new.index_select(0, idx).contiguous(),
                                 self.slot_mapping.index_select(0, idx).contiguous())
        k_new, v_new, slots = self._append_rows
        return paged_decode_append(self.q_decode, k_new, v_new, self.k_cache, self.v_cache,
                                   slots, self.decode_tables, self.context_lens,
                                   p.max_context_len, self.wl.scale,
                                   num_workers=self.num_workers, out=self.out_decode,
                                   workspace=self.workspace)

    def run_appended(self):
        self.decode_append()
        return self

    def mixed(self):
        """Prefill and decode of the step in one call (one launch for the common shapes)."""
        if self.q_prefill is None or self.q_decode is None:
            self.prefill()
            self.decode()
            return
        p = self.plan
        mixed_attention(self.k_cache, self.v_cache, self.wl.scale, self.q_prefill,
                        self.cu_seqlens_q, self.cu_seqlens_k, self.prefill_tables,
                        p.max_seqlen_q, p.max_seqlen_k, self.q_decode, self.decode_tables,
                        self.context_lens, p.max_context_len, num_workers=self.num_workers,
                        out_prefill=self.out_prefill, out_decode=self.out_decode,
                        workspace=self.workspace, rotary=self.rotary)

    def run_mixed(self):
        self.store()
        self.mixed()
        return self

    def outputs_numpy(self) -> dict:
        """Outputs as float64 numpy (bf16 widened exactly)."""
        out = {}
        for key, t in (("prefill", self.q_prefill is not None and self.out_prefill),
                       ("decode", self.q_decode is not None and self.out_decode)):
            if t is False or t is None:
                continue
            out[key] = t.detach().float().cpu().numpy().astype(np.float64)
        return out
