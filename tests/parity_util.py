"""Shared helpers for the GPU parity tests: tolerances and edge-case workloads."""
from __future__ import annotations

import numpy as np

import workloads
from workloads import SeqSpec as S

# match criteria: bf16 in / fp32 accumulate, and pure fp32
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def assert_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str) -> dict:
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if got.size == 0:
        return {"max": 0.0, "mean": 0.0}
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    stats = {"max": float(err.max()), "mean": float(err.mean())}
    if dtype == "f32":
        assert stats["max"] <= F32_MAX_ABS, f"{what}: {stats}"
    else:
        assert stats["max"] <= BF16_MAX_ABS and stats["mean"] <= BF16_MEAN_ABS, f"{what}: {stats}"
    return stats


def edge_workloads(seed: int = 0):
    """Ragged tails, one-token contexts, empty prompts, prefix sharing, every grouping
    ratio the kernels specialise (1, 2, 3, 4, 8, 16) and both head dims."""
    return [
        workloads.custom("edge_gqa4_d128_bs16", "bf16", 8, 2, 128, 16,
                         [S("prefill", 37, 37), S("prefill", 70, 5), S("decode", 300, 1),
                          S("decode", 1, 1), S("prefill", 1, 1), S("prefill", 16, 0),
                          S("decode", 17, 1)], seed=seed),
        workloads.custom("edge_mha_d64_bs4", "bf16", 3, 3, 64, 4,
                         [S("decode", 9, 1), S("prefill", 130, 130), S("prefill", 66, 63),
                          S("decode", 64, 1), S("decode", 65, 1)], seed=seed + 1),
        workloads.custom("edge_f32_gqa2_d128_bs8", "f32", 4, 2, 128, 8,
                         [S("prefill", 45, 45), S("decode", 33, 1), S("prefill", 90, 2),
                          S("decode", 2, 1)], seed=seed + 2),
        workloads.custom("edge_f32_mha_d64_bs32", "f32", 2, 2, 64, 32,
                         [S("prefill", 100, 100), S("decode", 31, 1), S("decode", 97, 1)],
                         seed=seed + 3),
        workloads.custom("edge_prefix_g8_bs256", "bf16", 16, 2, 128, 256,
                         [S("prefill", 512 + 130, 130, 0, 512), S("prefill", 513, 1, 0, 512),
                          S("prefill", 768 + 64, 64, 0, 512), S("decode", 513, 1)],
                         seed=seed + 4),
        workloads.custom("edge_long_g8_bs256", "bf16", 16, 2, 128, 256,
                         [S("decode", 2049, 1), S("decode", 255, 1), S("decode", 256, 1),
                          S("decode", 257, 1), S("prefill", 700, 700)], seed=seed + 5),
        workloads.custom("edge_g16_d64_bs32", "bf16", 32, 2, 64, 32,
                         [S("decode", 100, 1), S("prefill", 77, 77), S("decode", 1000, 1)],
                         seed=seed + 6),
        workloads.custom("edge_g3_d128_bs64", "bf16", 6, 2, 128, 64,
                         [S("decode", 129, 1), S("prefill", 200, 200), S("decode", 64, 1)],
                         seed=seed + 7),
    ]
