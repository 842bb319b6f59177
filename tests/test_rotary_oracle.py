"""Pins of the oracle's rotary position embedding (oracle/rotary.py) against what the
definition fixes (RoFormer's rotation of dimension pairs, half-split pairing), not
against a retyped formula: the identity at position 0, one hand-worked rotation,
pair norms, inverse and composition, the relative-position property of the scores,
and round-to-nearest-even on hand-picked ties.  No GPU."""
import math

import numpy as np

from oracle import rotary as R


def test_position_zero_is_the_identity():
    x = np.random.default_rng(0).standard_normal((5, 3, 64))
    assert np.array_equal(R.rotate(x, np.zeros(5)), x)


def test_hand_worked_rotation_of_the_first_pair():
    # D = 4: pairs (0, 2) and (1, 3), frequencies 1 and base^(-1/2) = 0.01
    x = np.array([[1.0, 0.0, 0.0, 0.0]])
    got = R.rotate(x, [2.0])
    assert np.allclose(got, [[math.cos(2.0), 0.0, math.sin(2.0), 0.0]], atol=1e-15)
    y = np.array([[0.0, 1.0, 0.0, 0.0]])
    got = R.rotate(y, [100.0])  # angle 100 * 0.01 = 1 on the second pair
    assert np.allclose(got, [[0.0, math.cos(1.0), 0.0, math.sin(1.0)]], atol=1e-13)


def test_each_pair_keeps_its_length():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 2, 128))
    y = R.rotate(x, rng.integers(0, 5000, 7))
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)


def test_inverse_and_composition():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 64))
    p = rng.integers(0, 3000, 6).astype(np.float64)
    q = rng.integers(0, 3000, 6).astype(np.float64)
    assert np.allclose(R.rotate(R.rotate(x, p), -p), x, atol=1e-12)
    assert np.allclose(R.rotate(R.rotate(x, p), q), R.rotate(x, p + q), atol=1e-10)


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((1, 128))
    for d in (0, 1, 7, 300):
        s1 = (R.rotate(q, [1000.0 + d]) * R.rotate(k, [1000.0])).sum()
        s2 = (R.rotate(q, [d]) * R.rotate(k, [0.0])).sum()
        assert math.isclose(s1, s2, rel_tol=1e-9, abs_tol=1e-9)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even (1.0) wins; 1 + 3*2^-8 rounds up
    # to 1 + 2^-6 (even); just above the tie rounds up
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -30, -2.5])
    want = np.array([0x3F80, 0x3F82, 0x3F81, 0xC020], np.uint16)
    assert np.array_equal(R.round_to_bf16(x), want)
