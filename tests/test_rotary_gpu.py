"""Rotary position embedding fused into the KV write and the attention calls, on the
GPU through the C ABI, against the oracle (oracle/rotary.py):

* the rotary KV write: V bit for bit, K within one unit in the last place of the
  cache type (the GPU rotates in fp32 with an fp32 table, the oracle in float64; both
  round once to nearest even) and bit-exact for all but a sliver of elements; slots
  not written keep their poison;
* whole steps (prefill and decode, bf16 on the MFMA / streaming kernels and fp32 on
  the generic one) with K rotated on write and queries rotated in the kernels'
  prologue, at the usual tolerances."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from oracle import rotary as R
from parity_util import assert_close
from workloads import SeqSpec as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_store_rotary(dtype, d):
    import paged_kv_cache_437_amd as pkv
    from paged_kv_cache_437_amd.step import STALE_BITS, to_device_values
    rng = np.random.default_rng(7)
    n, hkv, nb, bs = 300, 4, 40, 16
    vals = lambda: rng.standard_normal((n, hkv, d)).astype(np.float32)
    k, v = vals(), vals()
    if dtype == "bf16":
        k, v = workloads.round_to_bf16_bits(k), workloads.round_to_bf16_bits(v)
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[5] = -1  # a padding row
    pos = rng.integers(0, 4000, n).astype(np.int32)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.empty((nb, bs, hkv, d), dtype=dt, device="cuda")
    vc = torch.empty_like(kc)
    for c in (kc, vc):
        if dtype == "bf16":
            c.view(torch.int16).fill_(STALE_BITS["nan"]["bf16"])
        else:
            c.view(torch.int32).fill_(STALE_BITS["nan"]["f32"])
    table = pkv.rotary_table(4096, d)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    pkv.store_kvcache(to_device_values(k, "cuda"), to_device_values(v, "cuda"), kc, vc, i32(slots),
                      positions=i32(pos), rotary=table)
    torch.cuda.synchronize()
    raw = np.uint16 if dtype == "bf16" else np.uint32
    view = torch.int16 if dtype == "bf16" else torch.int32
    got_k = kc.view(view).cpu().numpy().view(raw).reshape(nb * bs, hkv, d)
    got_v = vc.view(view).cpu().numpy().view(raw).reshape(nb * bs, hkv, d)
    rot = R.rotate(oracle.as_float(k), pos)
    want_k = R.round_to_bf16(rot) if dtype == "bf16" else rot.astype(np.float32).view(np.uint32)
    v_bits = v if dtype == "bf16" else v.view(np.uint32)
    written = slots >= 0
    assert np.array_equal(got_v[slots[written]], v_bits[written])
    gk, wk = got_k[slots[written]].astype(np.int64), want_k[written].astype(np.int64)
    if dtype == "bf16":
        assert np.abs(gk - wk).max() <= 1, "K more than one bf16 ulp from the oracle"
        assert (gk != wk).mean() < 2e-3
    else:
        gf = got_k[slots[written]].view(np.float32)
        assert np.abs(gf.astype(np.float64) - rot[written]).max() <= 1e-5
    untouched = np.setdiff1d(np.arange(nb * bs), slots[written])
    stale = STALE_BITS["nan"][dtype]
    assert (got_k[untouched] == stale).all() and (got_v[untouched] == stale).all()


def _rotary_workloads():
    return [
        workloads.custom("rot_bf16_gqa2_d128_bs16", "bf16", 8, 4, 128, 16,
                         [S("prefill", 150, 150), S("decode", 300, 1), S("prefill", 90, 30),
                          S("decode", 1, 1), S("decode", 1025, 1)], seed=21),
        workloads.custom("rot_bf16_mha_d64_bs256", "bf16", 4, 4, 64, 256,
                         [S("prefill", 700, 700), S("decode", 513, 1), S("prefill", 300, 44)],
                         seed=22),
        workloads.custom("rot_f32_gqa2_d128_bs8", "f32", 4, 2, 128, 8,
                         [S("prefill", 45, 45), S("decode", 33, 1), S("prefill", 90, 2)],
                         seed=23),
        workloads.custom("rot_f32_mha_d64_bs32", "f32", 2, 2, 64, 32,
                         [S("prefill", 100, 100), S("decode", 97, 1)], seed=24),
        # prefill q tiles of 32 and 16 tokens (4 and 8 q heads per kv head), head_dim 64
        # and 128, whose cos/sin rows the kernel stages in LDS
        workloads.custom("rot_bf16_gqa4_d64_bs64", "bf16", 8, 2, 64, 64,
                         [S("prefill", 333, 333), S("prefill", 70, 20), S("decode", 129, 1)],
                         seed=25),
        workloads.custom("rot_bf16_gqa8_d128_bs256", "bf16", 16, 2, 128, 256,
                         [S("prefill", 599, 599), S("prefill", 17, 17), S("decode", 600, 1)],
                         seed=26),
        # 2 q heads per kv head at head_dim 128 with blocks of 256 keys (the varlen
        # prefill's shape): q tiles of 64 tokens, whose table rows fill both second K/V
        # buffers, loaded ahead of tile 0; a partial last q tile and a cached prefix
        workloads.custom("rot_bf16_gqa2_d128_bs256", "bf16", 16, 8, 128, 256,
                         [S("prefill", 700, 700), S("prefill", 1000, 300), S("decode", 513, 1)],
                         seed=27),
        # more than 64 sequences: the item search finds sequences past the first 64,
        # whose bounds it loads after the search
        workloads.custom("rot_bf16_gqa2_d128_bs64_many", "bf16", 4, 2, 128, 64,
                         [S("prefill", 1 + (37 * i) % 90, 1 + (37 * i) % 90) for i in range(70)]
                         + [S("prefill", 200, 75), S("decode", 130, 1)], seed=28),
    ]


# table rows per case: the last case's table ends at its longest context, so the rows
# of the 599-token prompt's last q tile past its last token (positions 599..607) clamp to
# the table's last row
_TABLE_ROWS = [2048, 2048, 2048, 2048, 2048, 600, 2048, 2048]


@pytest.mark.parametrize("idx", range(8))
def test_rotary_step_parity(idx):
    import paged_kv_cache_437_amd as pkv
    from paged_kv_cache_437_amd.step import DeviceStep
    wl = _rotary_workloads()[idx]
    table = pkv.rotary_table(_TABLE_ROWS[idx], wl.head_dim)
    st = DeviceStep(wl, device="cuda", rotary=table).run()
    got = st.outputs_numpy()
    torch.cuda.synchronize()
    ref = oracle.run_step(R.rotary_step(wl))
    for key in ("prefill", "decode"):
        if key in ref:
            assert_close(got[key], ref[key], wl.dtype, f"{wl.name} {key}")
    # the rotation matters: without it the outputs differ well beyond the tolerance
    plain = oracle.run_step(wl)
    key = "prefill"
    assert np.abs(plain[key] - ref[key]).max() > 0.05
