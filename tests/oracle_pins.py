"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` raises AssertionError on a mismatch.  They reach the oracle only
through module attributes (``pa.<fn>``, ``bm.<fn>``, ``st.<fn>``) so that the
planted-mistake tests can swap one function for a wrong one and watch a pin fail.

What pins what (cited passages are in the fixture files and the oracle header):
* golden fixtures (hand-worked): KV write indexing, the attention definition
  (alignment, grouping, scale, normalisation), the block manager's allocation;
* brute force: pure-Python loops over the generator's contiguous, unpaged K/V,
  with its own bf16 decoding; covers write + gather + attention together;
* torch's CPU scaled_dot_product_attention in float64 (library routine, its own
  GQA grouping, a ``tril``-built bottom-right mask);
* closed forms: one visible key, equal keys, one-hot probes (bit-exact);
* invariants: block relabelling, private copies of a shared prefix, stale
  poisoning with NaN / Inf / 1e30, decode == last prefill row, suffix prefill ==
  tail rows, GQA == duplicated MHA, split-K merge == unsplit;
* float32 vs float64 agreement.
"""
from __future__ import annotations

import copy
import json
import math
import os
import struct

import numpy as np

import oracle.block_manager as bm
import oracle.paged_attention as pa
import oracle.step as st
import workloads
from workloads import SeqSpec

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- golden

def pin_golden_store():
    g = _load("store_kvcache_tiny.json")
    shape = (g["num_blocks"], g["block_size"], g["num_kv_heads"], g["head_dim"])
    kc = np.full(shape, g["stale"], np.int64)
    vc = np.full(shape, g["stale"], np.int64)
    pa.store_kvcache(kc, vc, np.array(g["k"]), np.array(g["v"]), g["slot_mapping"])
    assert kc.tolist() == g["k_cache"], "golden KV write: k_cache"
    assert vc.tolist() == g["v_cache"], "golden KV write: v_cache"


def pin_golden_attention():
    g = _load("attention_tiny.json")
    for case in g["cases"]:
        q, k, v = (np.array(case[x], np.float64) for x in ("q", "k", "v"))
        want = np.array(case["out"])
        got = pa.causal_attention(q, k, v, case["scale"])
        assert np.allclose(got, want, rtol=0, atol=1e-12), case["name"]
        # the same case through a paged cache: keys scattered over blocks of 1
        Lk, Hkv, D = k.shape
        kc = np.full((Lk + 2, 1, Hkv, D), np.nan)
        vc = np.full((Lk + 2, 1, Hkv, D), np.nan)
        table = [Lk + 1 - j for j in range(Lk)]  # reversed, leaving block 0 stale
        pa.store_kvcache(kc, vc, k, v, table)
        got = pa.paged_prefill(q, kc, vc, [0, q.shape[0]], [0, Lk], [table], case["scale"])
        assert np.allclose(got, want, rtol=0, atol=1e-12), case["name"] + " (paged)"


def pin_golden_block_manager():
    g = _load("block_manager_tiny.json")
    seqs = [SeqSpec(s["phase"], s["context_len"], s["new_tokens"], s.get("prefix_group", -1),
                    s.get("prefix_len", 0)) for s in g["seqs"]]
    wl = workloads.Workload("golden", "f32", 1, 1, 1, g["block_size"], g["num_blocks"],
                            np.array(g["free_order"]), 1.0, 0, seqs)
    plan = bm.plan_step(wl)
    assert plan["tables"] == g["tables"], "golden tables"
    assert {str(b): r for b, r in plan["ref_counts"].items()} == g["ref_counts"], "ref counts"
    assert [list(x) for x in plan["history_slots"]] == g["history_slots"], "history slots"
    assert [list(x) for x in plan["step_slots"]] == g["step_slots"], "step slots"
    assert plan["cu_seqlens_q"] == g["cu_seqlens_q"]
    assert plan["cu_seqlens_k"] == g["cu_seqlens_k"]
    assert plan["context_lens"] == g["context_lens"]
    # the same allocation step by step, then free sequence 3
    pool = bm.IdPool(g["num_blocks"], g["free_order"])
    tables = []
    for i, s in enumerate(seqs):
        t = []
        if i == 3:
            pool.retain(tables[2][0])
            t.append(tables[2][0])
        while len(t) < -(-s.context_len // g["block_size"]):
            t.append(pool.take())
        tables.append(t)
    assert list(pool.free_ids) == g["free_after"], "free queue after allocation"
    for b in tables[3]:
        pool.release(b)
    after = g["free_sequence_3"]
    assert list(pool.free_ids) == after["free_after"], "free queue after freeing seq 3"
    assert {str(b): r for b, r in pool.in_use().items()} == after["ref_counts"]
    # exhaustion: the pool is fixed, allocation fails instead of inventing ids
    while pool.take() is not None:
        pass
    assert pool.take() is None and len(pool.in_use()) == g["num_blocks"]


# ----------------------------------------------------------------------------- brute force

def _bf16_to_py(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _to_lists(a):
    if a.dtype == np.uint16:
        return [[[_bf16_to_py(x) for x in row] for row in tok] for tok in a]
    return a.astype(np.float64).tolist()


def brute_force_sequence(q, k, v, scale, hq, hkv):
    """Pure-Python softmax attention on contiguous rows (q [Lq][Hq][D], k/v [Lk][Hkv][D])."""
    serves = []  # kv head of each q head: kv head j serves hq/hkv consecutive q heads
    for j in range(hkv):
        serves += [j] * (hq // hkv)
    Lq, Lk = len(q), len(k)
    out = []
    for i in range(Lq):
        newest = Lk - Lq + i  # the i-th new token's position in the sequence
        row = []
        for h in range(hq):
            j = serves[h]
            scores = [scale * math.fsum(a * b for a, b in zip(q[i][h], k[t][j]))
                      for t in range(newest + 1)]
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            total = math.fsum(w)
            row.append([math.fsum(w[t] * v[t][j][d] for t in range(newest + 1)) / total
                        for d in range(len(q[i][h]))])
        out.append(row)
    return out


def tiny_workloads(seed):
    """Small workloads spanning the cases: GQA and MHA, f32 and bf16, ragged tails,
    history before the step, a shared prefix, single-token contexts."""
    mixes = [
        ("mix_gqa_f32", "f32", 4, 2, 8, 4,
         [SeqSpec("prefill", 7, 7), SeqSpec("prefill", 10, 3), SeqSpec("decode", 9, 1),
          SeqSpec("decode", 1, 1), SeqSpec("prefill", 1, 1)]),
        ("mix_mha_bf16", "bf16", 2, 2, 16, 4,
         [SeqSpec("decode", 13, 1), SeqSpec("prefill", 6, 6), SeqSpec("prefill", 4, 0),
          SeqSpec("decode", 4, 1)]),
        ("prefix_bf16", "bf16", 4, 1, 8, 4,
         [SeqSpec("prefill", 11, 3, 0, 8), SeqSpec("prefill", 13, 5, 0, 8),
          SeqSpec("decode", 6, 1)]),
    ]
    return [workloads.custom(n, dt, hq, hkv, d, bs, seqs, seed=seed)
            for (n, dt, hq, hkv, d, bs, seqs) in mixes]


def pin_brute_force(seed=0):
    for wl in tiny_workloads(seed):
        res = st.run_step(wl)
        plan = res["plan"]
        row = 0
        for i in plan["prefill"]:
            s = wl.seqs[i]
            want = brute_force_sequence(_to_lists(wl.q[i]), _to_lists(wl.k[i]),
                                        _to_lists(wl.v[i]), wl.scale, wl.num_q_heads,
                                        wl.num_kv_heads)
            got = res["prefill"][row:row + s.new_tokens]
            assert np.allclose(got, np.array(want).reshape(got.shape), rtol=0, atol=1e-12), \
                f"{wl.name} prefill seq {i}"
            row += s.new_tokens
        for n, i in enumerate(plan["decode"]):
            want = brute_force_sequence(_to_lists(wl.q[i]), _to_lists(wl.k[i]),
                                        _to_lists(wl.v[i]), wl.scale, wl.num_q_heads,
                                        wl.num_kv_heads)
            assert np.allclose(res["decode"][n], np.array(want)[0], rtol=0, atol=1e-12), \
                f"{wl.name} decode seq {i}"


def pin_sdpa(seed=0):
    import torch
    import torch.nn.functional as F

    def widen(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.astype(np.int32) << 16).view(torch.float32).double()
        return torch.from_numpy(a).double()

    for wl in tiny_workloads(seed + 100):
        res = st.run_step(wl)
        plan = res["plan"]
        outs = {"prefill": [], "decode": []}
        for phase in ("prefill", "decode"):
            for i in plan[phase]:
                s = wl.seqs[i]
                q = widen(wl.q[i]).permute(1, 0, 2)[None]
                k = widen(wl.k[i]).permute(1, 0, 2)[None]
                v = widen(wl.v[i]).permute(1, 0, 2)[None]
                Lq, Lk = s.new_tokens, s.context_len
                mask = torch.ones(Lq, Lk, dtype=torch.bool).tril(diagonal=Lk - Lq)
                if Lq == 0:
                    outs[phase].append(np.zeros((0, wl.num_q_heads, wl.head_dim)))
                    continue
                o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=wl.scale,
                                                   enable_gqa=True)
                outs[phase].append(o[0].permute(1, 0, 2).numpy())
        if plan["prefill"]:
            got = res["prefill"]
            want = np.concatenate(outs["prefill"])
            assert np.allclose(got, want, rtol=0, atol=1e-12), f"{wl.name} prefill vs SDPA"
        if plan["decode"]:
            want = np.concatenate(outs["decode"])
            assert np.allclose(res["decode"], want, rtol=0, atol=1e-12), f"{wl.name} decode vs SDPA"


# ----------------------------------------------------------------------------- closed forms

def pin_one_key():
    wl = workloads.custom("one_key", "f32", 2, 1, 8, 4,
                          [SeqSpec("prefill", 1, 1), SeqSpec("decode", 1, 1)], seed=3)
    res = st.run_step(wl)
    assert np.array_equal(res["prefill"][0], np.repeat(wl.v[0][0].astype(np.float64), 2, 0))
    assert np.array_equal(res["decode"][0], np.repeat(wl.v[1][0].astype(np.float64), 2, 0))


def pin_equal_keys():
    wl = workloads.custom("equal_keys", "f32", 2, 2, 8, 4,
                          [SeqSpec("prefill", 9, 4), SeqSpec("decode", 7, 1)], seed=4)
    for i in range(2):
        wl.k[i][:] = wl.k[i][0]
    res = st.run_step(wl)
    for r in range(4):  # prefill row r sees keys 0 .. 5 + r
        visible = wl.v[0][:6 + r].astype(np.float64)
        mean = np.array([[math.fsum(visible[:, h, d]) / len(visible) for d in range(8)]
                         for h in range(2)])
        assert np.allclose(res["prefill"][r], mean, rtol=0, atol=1e-12), f"equal keys row {r}"
    visible = wl.v[1].astype(np.float64)
    mean = np.array([[math.fsum(visible[:, h, d]) / 7 for d in range(8)] for h in range(2)])
    assert np.allclose(res["decode"][0], mean, rtol=0, atol=1e-12)


def one_hot_probe(wl, seq, target, dim=0, big=256.0, key_scale=32.0):
    """Make sequence ``seq`` attend to exactly one key: zero every key, put a power
    of two at ``dim`` of key ``target`` and of every query row; the score gap
    (big * key_scale * scale) makes every other weight exp(-gap) == 0.0."""
    enc = (lambda x: x) if wl.dtype == "f32" else (lambda x: workloads.round_to_bf16_bits(
        np.asarray(x, np.float32)))
    wl.k[seq][:] = enc(np.zeros(wl.k[seq].shape, np.float32))
    kk = np.zeros(wl.k[seq].shape[1:], np.float32)
    kk[:, dim] = key_scale
    wl.k[seq][target] = enc(kk)
    qq = np.zeros(wl.q[seq].shape, np.float32)
    qq[:, :, dim] = big
    wl.q[seq][:] = enc(qq)


def pin_one_hot():
    seqs = [SeqSpec("decode", 23, 1), SeqSpec("decode", 23, 1), SeqSpec("decode", 23, 1),
            SeqSpec("prefill", 23, 2)]
    wl = workloads.custom("probe", "bf16", 4, 2, 16, 8, seqs, seed=5, scale=0.25)
    targets = [0, 7, 8, 22]  # first key, last of block 0, first of block 1, the newest key
    for i, t in enumerate(targets):
        one_hot_probe(wl, i, t)
    res = st.run_step(wl)
    for n, i in enumerate(res["plan"]["decode"]):
        want = pa.bf16_bits_to_float(wl.v[i][targets[i]])
        want = np.repeat(want, 2, axis=0)  # 4 q heads over 2 kv heads
        assert np.array_equal(res["decode"][n], want), f"one-hot probe seq {i}"
    want = np.repeat(pa.bf16_bits_to_float(wl.v[3][22]), 2, axis=0)
    # prefill rows sit at positions 21 and 22: row 0 cannot see key 22 (all its keys are 0)
    assert np.array_equal(res["prefill"][1], want), "one-hot probe on the newest prefill row"


# ----------------------------------------------------------------------------- invariants

def pin_relabel_invariance(seed=0):
    for wl in tiny_workloads(seed + 7):
        a = st.run_step(wl)
        wl2 = copy.copy(wl)
        wl2.num_blocks = wl.num_blocks + 5
        wl2.free_order = np.random.default_rng(seed + 99).permutation(wl2.num_blocks)
        b = st.run_step(wl2)
        assert a["plan"]["tables"] != b["plan"]["tables"]
        for key in ("prefill", "decode"):
            if key in a:
                assert np.array_equal(a[key], b[key]), f"{wl.name}: relabelling changed {key}"


def pin_prefix_copy_invariance(seed=0):
    wl = tiny_workloads(seed)[2]
    shared = st.run_step(wl)
    wl2 = copy.copy(wl)
    wl2.seqs = [SeqSpec(s.phase, s.context_len, s.new_tokens) for s in wl.seqs]
    wl2.num_blocks = wl.num_blocks + 8
    wl2.free_order = np.arange(wl2.num_blocks)[::-1].copy()
    private = st.run_step(wl2)
    ids = shared["plan"]["tables"]
    assert ids[0][:2] == ids[1][:2] and private["plan"]["tables"][0][:2] != \
        private["plan"]["tables"][1][:2]
    for key in ("prefill", "decode"):
        assert np.array_equal(shared[key], private[key]), f"shared vs copied prefix: {key}"


def pin_stale_invariance(seed=0):
    for wl in tiny_workloads(seed + 11):
        if wl.dtype == "f32":
            fills = [np.float32(np.nan), np.float32(np.inf), np.float32(-np.inf), np.float32(1e30)]
        else:
            fills = [np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80), np.uint16(0x7149)]
        outs = [st.run_step(wl, stale=f) for f in fills]
        for key in ("prefill", "decode"):
            if key in outs[0]:
                assert np.isfinite(outs[0][key]).all(), f"{wl.name}: stale value leaked"
                for o in outs[1:]:
                    assert np.array_equal(outs[0][key], o[key]), f"{wl.name}: stale leak"


def pin_decode_equals_last_prefill_row(seed=0):
    L = 19
    wl = workloads.custom("dec_vs_pre", "bf16", 4, 2, 16, 4,
                          [SeqSpec("prefill", L, L), SeqSpec("decode", L, 1),
                           SeqSpec("prefill", L, 6)], seed=seed + 21)
    for i in (1, 2):
        wl.k[i] = wl.k[0].copy()
        wl.v[i] = wl.v[0].copy()
    wl.q[1] = wl.q[0][-1:].copy()
    wl.q[2] = wl.q[0][-6:].copy()
    res = st.run_step(wl)
    assert np.allclose(res["decode"][0], res["prefill"][L - 1], rtol=0, atol=1e-13)
    assert np.allclose(res["prefill"][L:L + 6], res["prefill"][L - 6:L], rtol=0, atol=1e-13)


def pin_gqa_equals_duplicated_mha(seed=0):
    seqs = [SeqSpec("prefill", 9, 9), SeqSpec("decode", 14, 1)]
    g = workloads.custom("gqa", "f32", 4, 2, 8, 4, seqs, seed=seed + 31)
    m = workloads.custom("mha", "f32", 4, 4, 8, 4, seqs, seed=seed + 31)
    for i in range(2):
        m.q[i] = g.q[i].copy()
        m.k[i] = np.repeat(g.k[i], 2, axis=1)  # kv heads 0,0,1,1
        m.v[i] = np.repeat(g.v[i], 2, axis=1)
    a, b = st.run_step(g), st.run_step(m)
    for key in ("prefill", "decode"):
        assert np.array_equal(a[key], b[key]), f"GQA vs duplicated MHA: {key}"


def pin_split_merge(seed=0):
    rng = np.random.default_rng(seed + 41)
    for L, cuts in ((37, [0, 16, 32, 37]), (64, [0, 16, 32, 48, 64]), (5, [0, 5]),
                    (33, [0, 1, 2, 33])):
        q = rng.standard_normal((4, 8))
        k = rng.standard_normal((L, 2, 8)) * 3
        v = rng.standard_normal((L, 2, 8))
        m, l, o = pa.decode_split_partials(q, k, v, 0.35, cuts)
        got = pa.combine_partials(m, l, o)
        want = brute_force_sequence(q[None].tolist(), k.tolist(), v.tolist(), 0.35, 4, 2)[0]
        assert np.allclose(got, np.array(want), rtol=0, atol=1e-12), f"split merge L={L}"


def pin_fp32_close_to_fp64(seed=0):
    wl = workloads.tiny_mixed(seed)
    a = st.run_step(wl, dtype=np.float64)
    b = st.run_step(wl, dtype=np.float32)
    for key in ("prefill", "decode"):
        assert np.abs(a[key] - b[key]).max() <= 1e-6, f"fp32 vs fp64 {key}"


ALL_PINS = [
    pin_golden_store, pin_golden_attention, pin_golden_block_manager, pin_brute_force, pin_sdpa,
    pin_one_key, pin_equal_keys, pin_one_hot, pin_relabel_invariance, pin_prefix_copy_invariance,
    pin_stale_invariance, pin_decode_equals_last_prefill_row, pin_gqa_equals_duplicated_mha,
    pin_split_merge, pin_fp32_close_to_fp64,
]
