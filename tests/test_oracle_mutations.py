"""Planted mistakes in the oracle (CPU only) must each trip a pin.

Each case patches one oracle function with a plausible error and checks that
the corresponding pin test fails; the patched oracle is restored afterwards.
"""

import numpy as np
import pytest

import oracle
import oracle.mla as om
import test_oracle_decode as td
import test_oracle_rope as tr


def _rope_wrong_sign(x, pos, base):
    return om.__dict__["_real_rope"](x, -np.asarray(pos), base)


def _rope_rotate_half(x, pos, base):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * om.rope_theta(d, base)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * np.cos(ang) - b * np.sin(ang),
                           a * np.sin(ang) + b * np.cos(ang)], axis=-1)


def _expand_transposed(c, w_uk_h, w_uv_h):
    # reads the weight as if it were stored [d_c, d_nope]
    return c @ w_uk_h.reshape(w_uk_h.shape[1], w_uk_h.shape[0]), c @ w_uv_h.T


def _expand_key_sign(c, w_uk_h, w_uv_h):
    return -(c @ w_uk_h.T), c @ w_uv_h.T


def _gather_off_by_one(kv_latent, kv_rope, block_table, b, length, page_size):
    t = np.arange(length)
    pages = np.asarray(block_table)[b, (t + 1) // page_size % block_table.shape[1]]
    return kv_latent[pages, t % page_size, :], kv_rope[pages, t % page_size, :]


CASES = [
    ("apply_rope", _rope_wrong_sign, [tr.test_two_dims_rotate_by_position_radians]),
    ("apply_rope", _rope_rotate_half, [tr.test_four_dims_adjacent_pairs_closed_form]),
    ("expand_kv", _expand_transposed, [td.test_oracle_matches_torch_sdpa]),
    ("expand_kv", _expand_key_sign, [td.test_oracle_matches_torch_sdpa]),
    ("gather_cache", _gather_off_by_one, [td.test_oracle_matches_torch_sdpa]),
]


@pytest.mark.parametrize("name,bad,pins", CASES, ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, bad, pins):
    om.__dict__.setdefault("_real_rope", om.apply_rope)
    monkeypatch.setattr(om, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


def test_planted_softmax_scale_mistake_is_caught(monkeypatch):
    real = om._decode

    def bad(inputs, rows, return_probs, absorbed):
        inputs = dict(inputs)
        inputs["softmax_scale"] = inputs["softmax_scale"] * 2
        return real(inputs, rows, return_probs, absorbed)

    monkeypatch.setattr(om, "_decode", bad)
    with pytest.raises(AssertionError):
        td.test_oracle_matches_torch_sdpa()


def test_planted_causal_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(om, "_visible", lambda length, q_len, j, causal: (length - q_len + j, length))
    with pytest.raises(AssertionError):
        td.test_mtp_first_token_equals_single_token_at_shorter_length()
