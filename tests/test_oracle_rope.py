"""Pins for the oracle's rotary embedding.

The rotary page ("Deepseek-V3 Define 1: Higher Attachment of Head" on
dataforcee.us, rotary-embedding part) groups coordinates into adjacent pairs and
rotates each pair by an angle proportional to the position; the latent-cache
page ("Multi-Head Latent Attention – Latent KV-Cache", "Residual & RoPE
Explanation") states that scores then depend only on relative distance.
"""

import numpy as np
import pytest

import oracle


def test_two_dims_rotate_by_position_radians():
    # one pair: theta_0 = base^0 = 1, so position p rotates by exactly p radians
    for p in [0, 1, 2, 7, 100]:
        for base in [10000.0, 2.0]:
            got = oracle.apply_rope(np.array([1.0, 0.0]), p, base)
            assert np.allclose(got, [np.cos(p), np.sin(p)], atol=1e-15, rtol=0)
            got = oracle.apply_rope(np.array([0.0, 1.0]), p, base)
            assert np.allclose(got, [-np.sin(p), np.cos(p)], atol=1e-15, rtol=0)


def test_four_dims_adjacent_pairs_closed_form():
    base = 10000.0
    th1 = base ** (-2.0 * 1 / 4)        # second pair's frequency
    p = 3
    e0 = oracle.apply_rope(np.array([1.0, 0, 0, 0]), p, base)
    assert np.allclose(e0, [np.cos(p), np.sin(p), 0, 0], atol=1e-15)
    e2 = oracle.apply_rope(np.array([0, 0, 1.0, 0]), p, base)
    assert np.allclose(e2, [0, 0, np.cos(p * th1), np.sin(p * th1)], atol=1e-15)
    e3 = oracle.apply_rope(np.array([0, 0, 0, 1.0]), p, base)
    assert np.allclose(e3, [0, 0, -np.sin(p * th1), np.cos(p * th1)], atol=1e-15)


def test_theta_ladder():
    th = oracle.rope_theta(64, 10000.0)
    assert th.shape == (32,)
    assert th[0] == 1.0
    assert np.allclose(th[1:] / th[:-1], 10000.0 ** (-2.0 / 64), rtol=1e-14)


def test_position_zero_is_identity_and_rotation_is_orthogonal():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(oracle.apply_rope(x, 0, 10000.0), x)
    y = oracle.apply_rope(x, 12345, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("d", [2, 16, 64])
def test_scores_depend_only_on_relative_position(d):
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for p, t, delta in [(10, 3, 5), (4096, 17, 1000), (0, 9, 31)]:
        a = oracle.apply_rope(q, p, 10000.0) @ oracle.apply_rope(k, t, 10000.0)
        b = oracle.apply_rope(q, p + delta, 10000.0) @ oracle.apply_rope(k, t + delta, 10000.0)
        assert abs(a - b) <= 1e-11 * max(1.0, abs(a))


def test_batched_positions_broadcast():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 8))
    pos = np.array([0, 5, 77])
    got = oracle.apply_rope(x, pos, 500.0)
    for i in range(3):
        assert np.allclose(got[i], oracle.apply_rope(x[i], pos[i], 500.0), atol=0, rtol=0)
