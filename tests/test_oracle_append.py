"""Pins of the cache-append oracle (oracle/append.py) against closed forms and
a placement case worked out by hand; RoPE and the e4m3 codec are pinned in
their own test files."""

import numpy as np
import pytest

import oracle


def test_rms_norm_of_a_constant_vector():
    # x = c * 1 (d entries): mean(x^2) = c^2, so y = c / sqrt(c^2 + eps) * g
    c, eps, d = 0.37, 1e-6, 24
    g = np.linspace(0.5, 1.5, d)
    y = oracle.rms_norm(np.full(d, c), g, eps)
    assert np.allclose(y, c / np.sqrt(c * c + eps) * g, rtol=1e-15, atol=0)


def test_rms_norm_output_rms_and_scale_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 512))
    ms = np.mean(x * x, axis=-1)
    # unit gain: mean(y^2) = ms / (ms + eps)
    y = oracle.rms_norm(x, np.ones(512), 1e-6)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-6), rtol=1e-13)
    # eps = 0: positive scaling of the input does not change the output
    y0 = oracle.rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(oracle.rms_norm(37.5 * x, np.ones(512), 0.0), y0, rtol=1e-13)
    # the gain multiplies coordinate by coordinate
    g = rng.uniform(0.5, 2.0, 512)
    assert np.allclose(oracle.rms_norm(x, g, 1e-6), y * g, rtol=1e-14)


def test_placement_worked_by_hand():
    # page size 4, two new tokens per sequence; lengths already count them
    table = np.array([[7, 2, 9], [5, 0, 0], [1, 3, 8]])
    seqlens = [5, 1, 12]
    pos, page, slot = oracle.append_positions(seqlens, 2, table, 4)
    # sequence 0: positions 3, 4 -> page 7 slot 3, page 2 slot 0
    # sequence 1: positions -1 (not written), 0 -> page 5 slot 0
    # sequence 2: positions 10, 11 -> page 8 slots 2, 3
    assert pos.tolist() == [[3, 4], [-1, 0], [10, 11]]
    assert page.tolist() == [[7, 2], [-1, 5], [8, 8]]
    assert slot.tolist() == [[3, 0], [-1, 0], [2, 3]]


def test_token_quantiser_bounds_and_zero_row():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((6, 512)) * rng.uniform(0.01, 10.0, (6, 1))
    codes, s = oracle.quantize_token_e4m3(y)
    back = oracle.e4m3_bits_to_f64(codes) * s[:, None]
    # the largest magnitude maps to 448 exactly; e4m3 keeps 3 fraction bits,
    # so nearest rounding is within 2^-4 relative for normal codes and
    # within half the subnormal step 2^-9 * s otherwise
    assert np.allclose(np.max(np.abs(back), axis=-1), np.max(np.abs(y), axis=-1), rtol=1e-15)
    err = np.abs(back - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-12))
    z_codes, z_s = oracle.quantize_token_e4m3(np.zeros(8))
    assert z_s == 1.0 and np.all(z_codes == 0)


def test_append_rotates_at_the_token_position():
    # the stored rotary key is RoPE at the token's own position: for a key
    # (1, 0) in pair i the rotated pair is (cos, sin) of pos * theta_i
    rng = np.random.default_rng(13)
    table = np.arange(12).reshape(3, 4)
    kv_c = rng.standard_normal((3, 2, 16))
    kr = np.zeros((3, 2, 8))
    kr[..., 0::2] = 1.0
    out = oracle.append_kv(kv_c, kr, np.ones(16), [9, 2, 14], 2, table, 4, 10000.0)
    theta = 10000.0 ** (-2.0 * np.arange(4) / 8)
    for b, L in enumerate([9, 2, 14]):
        for j in range(2):
            p = L - 2 + j
            assert np.allclose(out["kr"][b, j, 0::2], np.cos(p * theta), rtol=0, atol=1e-15)
            assert np.allclose(out["kr"][b, j, 1::2], np.sin(p * theta), rtol=0, atol=1e-15)
