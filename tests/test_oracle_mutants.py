"""Planted mistakes in the oracle (on the CPU): each must make at least one pin fail.

A pin set that a dropped term, a wrong sign or index, or a swapped operand slips
through would not be worth trusting; every mutant below is one such plausible
slip, swapped into the oracle's module for the duration of one test.
"""
import numpy as np
import pytest

import oracle.block_manager as bm
import oracle.paged_attention as pa
import oracle.step as st
from oracle_pins import ALL_PINS


def _attention_variant(*, top_left=False, drop_scale=False, use_k_as_v=False, no_norm=False,
                       no_max=False):
    def causal_attention(q, k, v, scale, dtype=np.float64):
        Lq, Hq, D = q.shape
        Lk, Hkv, _ = k.shape
        out = np.zeros((Lq, Hq, D), dtype)
        if Lq == 0:
            return out
        shift = 0 if top_left else Lk - Lq
        sees = np.arange(Lk)[None, :] <= (shift + np.arange(Lq))[:, None]
        for h in range(Hq):
            kh = pa.kv_head_of(h, Hq, Hkv)
            qh = pa.as_float(q[:, h, :], dtype)
            kk = pa.as_float(k[:, kh, :], dtype)
            vv = kk if use_k_as_v else pa.as_float(v[:, kh, :], dtype)
            scores = qh @ kk.T
            if not drop_scale:
                scores = scores * dtype(scale)
            scores = np.where(sees, scores, -np.inf)
            p = np.exp(scores - (0 if no_max else scores.max(axis=1, keepdims=True)))
            if not no_norm:
                p = p / p.sum(axis=1, keepdims=True)
            out[:, h, :] = p @ vv
        return out
    return causal_attention


def _gather_swapped(cache, table_row, length):
    bs = cache.shape[1]
    rows = [cache[int(table_row[j % bs]) % cache.shape[0], (j // bs) % bs] for j in range(length)]
    return np.stack(rows) if rows else np.empty((0,) + cache.shape[2:], cache.dtype)


def _gather_reversed_blocks(cache, table_row, length):
    bs = cache.shape[1]
    nb = -(-length // bs)
    rows = [cache[int(table_row[nb - 1 - j // bs]), j % bs] for j in range(length)]
    return np.stack(rows) if rows else np.empty((0,) + cache.shape[2:], cache.dtype)


def _store_block_offset_swapped(k_cache, v_cache, k, v, slot_mapping):
    nb, bs = k_cache.shape[:2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot == -1:
            continue
        offset, block = divmod(slot, bs)
        k_cache[block % nb, offset % bs] = k[t]
        v_cache[block % nb, offset % bs] = v[t]


def _store_k_into_both(k_cache, v_cache, k, v, slot_mapping):
    nb, bs = k_cache.shape[:2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot == -1:
            continue
        b, o = divmod(slot, bs)
        k_cache[b, o] = k[t]
        v_cache[b, o] = k[t]


def _slot_of_wrong(table_row, position, block_size):
    return int(table_row[position // block_size]) * block_size + position // block_size


def _combine_unweighted_l(m, l, o):
    M = m.max(axis=0)
    w = np.exp(m - M[None, :])
    return (w[:, :, None] * o).sum(axis=0) / l.sum(axis=0)[:, None]


def _decode_drops_newest(q, k_cache, v_cache, block_tables, context_lens, scale, dtype=np.float64):
    out = np.zeros(q.shape, dtype)
    for b in range(q.shape[0]):
        L = max(1, int(context_lens[b]) - 1)
        K = pa.gather_tokens(k_cache, block_tables[b], L)
        V = pa.gather_tokens(v_cache, block_tables[b], L)
        out[b] = pa.causal_attention(q[b:b + 1], K, V, scale, dtype)[0]
    return out


class _LifoPool(bm.IdPool):
    def take(self):
        if not self.free_ids:
            return None
        b = self.free_ids.pop()
        self.refs[b] = 1
        return b


class _NoSharePool(bm.IdPool):
    def retain(self, b):
        pass


MUTANTS = {
    "gqa_interleaved": [(pa, "kv_head_of", lambda h, hq, hkv: h % hkv)],
    "causal_top_left": [(pa, "causal_attention", _attention_variant(top_left=True))],
    "scale_dropped": [(pa, "causal_attention", _attention_variant(drop_scale=True))],
    "k_used_as_v": [(pa, "causal_attention", _attention_variant(use_k_as_v=True))],
    "softmax_not_normalised": [(pa, "causal_attention", _attention_variant(no_norm=True))],
    "gather_block_offset_swapped": [(pa, "gather_tokens", _gather_swapped)],
    "gather_blocks_reversed": [(pa, "gather_tokens", _gather_reversed_blocks)],
    "store_block_offset_swapped": [(pa, "store_kvcache", _store_block_offset_swapped),
                                   (st, "store_kvcache", _store_block_offset_swapped)],
    "store_k_into_v": [(pa, "store_kvcache", _store_k_into_both),
                       (st, "store_kvcache", _store_k_into_both)],
    "slot_offset_wrong": [(bm, "slot_of", _slot_of_wrong)],
    "combine_l_unweighted": [(pa, "combine_partials", _combine_unweighted_l)],
    "decode_drops_newest_key": [(pa, "paged_decode", _decode_drops_newest),
                                (st, "paged_decode", _decode_drops_newest)],
    "free_list_lifo": [(bm, "IdPool", _LifoPool)],
    "prefix_share_not_counted": [(bm, "IdPool", _NoSharePool)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for module, attr, value in MUTANTS[name]:
        monkeypatch.setattr(module, attr, value)
    caught = []
    for pin in ALL_PINS:
        try:
            # a planted mistake may read the NaN-poisoned stale blocks: numpy's warning
            # about it is expected here, the pins' verdict is what counts
            with np.errstate(invalid="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, KeyError, RuntimeError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
