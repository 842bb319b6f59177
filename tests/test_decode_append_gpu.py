"""The decode step in one call (pkv_paged_decode_append) against the two calls it
replaces (pkv_store_kvcache, then pkv_paged_decode), through the C ABI.

Both paths start from the same cache contents (the history written at set-up, stale
blocks NaN-poisoned) and must leave the whole pool and the outputs bit-identical: the
appending kernel writes each new row itself and takes the new token's K and V from
registers, where the separate decode reads them back from the cache.  Cases cover the
appending kernel (bf16, one q head per kv head, blocks of at least one decode chunk:
every kv-heads-per-stream width at head_dim 64 and 128, contexts of 1 token and at chunk
and block edges, several worker counts) and the two-kernel path the entry point takes
otherwise (grouped heads, blocks shorter than a chunk, fp32 caches), checking which
kernels ran, and the oracle on one case.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity_util import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

S = workloads.SeqSpec


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_437_amd as pkv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv._lib.load()
    return pkv


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


def _both(pkv, wl, num_workers=0):
    """(separate, fused, step, kernels the fused call launched): separate and fused each
    a dict of out / k_cache / v_cache bits."""
    from paged_kv_cache_437_amd.step import DeviceStep
    st = DeviceStep(wl, device="cuda", stale="nan", num_workers=num_workers)
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()
    st.store()
    st.decode()
    torch.cuda.synchronize()
    sep = {"out": _bits(st.out_decode), "k": _bits(st.k_cache), "v": _bits(st.v_cache)}
    st.k_cache.copy_(k0)
    st.v_cache.copy_(v0)
    st.out_decode.zero_()
    pkv.timing_collect()
    pkv.timing_enable(True)
    try:
        st.decode_append()
    finally:
        pkv.timing_enable(False)
    names = set(pkv.timing_collect())
    torch.cuda.synchronize()
    fused = {"out": _bits(st.out_decode), "k": _bits(st.k_cache), "v": _bits(st.v_cache)}
    return sep, fused, st, names


def _lens(rng, n, lo, hi):
    return [int(x) for x in rng.integers(lo, hi + 1, n)]


CASES = {
    # name: (dtype, Hq, Hkv, D, block_size, context lengths, worker counts, one kernel)
    "mha_d128_mh2_bs256": ("bf16", 32, 32, 128, 256, [1, 7, 8, 9, 255, 256, 257, 600, 2049],
                           [0, 7], True),
    "mha_d128_mh1_bs16": ("bf16", 3, 3, 128, 16, [1, 15, 16, 17, 31, 32, 33, 400], [0, 4], True),
    "mha_d64_mh1_bs32": ("bf16", 5, 5, 64, 32, [1, 31, 32, 33, 64, 65, 700], [0, 3], True),
    "mha_d64_mh2_bs16": ("bf16", 6, 6, 64, 16, [1, 15, 16, 17, 250], [0, 5], True),
    "mha_d64_mh4_bs8": ("bf16", 8, 8, 64, 8, [1, 7, 8, 9, 16, 17, 300], [0, 9], True),
    "gqa4_d128_bs16_two_kernels": ("bf16", 32, 8, 128, 16, [1, 8, 15, 16, 17, 100, 333, 1000],
                                   [0, 61], False),
    "gqa2_d64_bs8_two_kernels": ("bf16", 8, 4, 64, 8, [1, 2, 7, 8, 9, 64, 65, 300], [0, 3], False),
    "mha_d128_bs4_two_kernels": ("bf16", 8, 8, 128, 4, [1, 3, 4, 5, 77], [0], False),
    "f32_two_kernels": ("f32", 8, 2, 64, 16, [1, 16, 17, 90], [0], False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_matches_store_then_decode(pkv, name):
    dtype, hq, hkv, d, bs, lens, workers, one_kernel = CASES[name]
    wl = workloads.custom("append_" + name, dtype, hq, hkv, d, bs,
                          [S("decode", L, 1) for L in lens], seed=21)
    for w in workers:
        sep, fused, _, names = _both(pkv, wl, w)
        assert ("paged_decode_append" in names) == one_kernel, f"{name}: launches {sorted(names)}"
        assert ("store_kvcache" in names) != one_kernel, f"{name}: launches {sorted(names)}"
        for key in ("k", "v"):
            assert torch.equal(sep[key], fused[key]), f"{name} W={w}: {key} cache differs"
        assert torch.equal(sep["out"], fused["out"]), f"{name} W={w}: outputs differ"


def test_append_large_random_batch(pkv):
    """64 sequences of U[1, 4096] tokens, 16/16 heads: many stream ends per worker and
    streams cut between workers."""
    rng = np.random.default_rng(5)
    wl = workloads.custom("append_batch", "bf16", 16, 16, 128, 256,
                          [S("decode", L, 1) for L in _lens(rng, 64, 1, 4096)], seed=22)
    sep, fused, _, names = _both(pkv, wl)
    assert "paged_decode_append" in names
    for key in ("k", "v", "out"):
        assert torch.equal(sep[key], fused[key]), key


def test_append_headline_workload_against_oracle(pkv):
    wl = workloads.decode_mha(seed=1)
    sep, fused, st, names = _both(pkv, wl)
    assert "paged_decode_append" in names
    for key in ("k", "v", "out"):
        assert torch.equal(sep[key], fused[key]), key
    ref = oracle.run_step(wl)
    assert_close(st.outputs_numpy()["decode"], ref["decode"], wl.dtype, "decode_append decode_mha")


def test_append_refuses_missing_rows(pkv):
    wl = workloads.custom("append_args", "bf16", 8, 8, 128, 16, [S("decode", 20, 1)], seed=3)
    from paged_kv_cache_437_amd.step import DeviceStep
    st = DeviceStep(wl, device="cuda")
    with pytest.raises(ValueError):
        pkv.paged_decode_append(st.q_decode, st.k_new[:0], st.v_new[:0], st.k_cache, st.v_cache,
                                st.slot_mapping, st.decode_tables, st.context_lens,
                                st.plan.max_context_len, wl.scale)
