"""Pins for the oracle's own storage codecs: torch's CPU casts as the library routine."""

import numpy as np
import torch

import oracle


def test_bf16_decode_every_code():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties: a bf16 value plus half of its last place
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -3e38, np.inf, -np.inf])])
    ours = oracle.f64_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2                      # 0x7F and 0xFF
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == oracle.E4M3_MAX == 448.0
    assert ours[0x01] == 2.0 ** -9             # smallest subnormal
    assert ours[0x08] == 2.0 ** -6             # smallest normal


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000) * 60.0
    x = x[np.abs(x) <= 448.0]
    # midpoints between neighbouring codes (ties go to the even code)
    pos = oracle.e4m3_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids, [0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    ours = oracle.f64_to_e4m3_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    out = oracle.f64_to_e4m3_bits(np.array([500.0, 1e9, -700.0, np.nan]))
    assert list(out) == [0x7E, 0x7E, 0xFE, 0x7F]


def test_row_quantiser_matches_torch_cast_and_bounds():
    """kernel_models.quantize_rows_e4m3 (the fp8 path's query rounding, a kernel
    model, not part of the oracle): the scale is the smallest power of two 2^k with
    max|row| / 2^k <= 448, codes equal torch's float8_e4m3fn cast of row / 2^k (an
    exact division), and every value is within half an e4m3 step."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    x[3] = 0.0
    x[5, 7] = -abs(x[5]).max() * 2          # a negative row maximum
    x[9] *= 448.0 / np.abs(x[9]).max()      # a row maximum of exactly 448 keeps scale 1
    import kernel_models
    got = kernel_models.quantize_rows_e4m3(x)
    amax = np.abs(x).max(axis=1, keepdims=True)
    k = np.ceil(np.log2(np.where(amax > 0, amax, 448.0) / 448.0))
    scale = np.where(amax > 0, 2.0 ** k, 1.0)
    assert scale[9, 0] == 1.0
    y = x / scale
    # the row maximum lands in (224, 448]
    assert np.all((np.abs(y).max(axis=1) > 224) | (amax[:, 0] == 0))
    assert np.all(np.abs(y).max(axis=1) <= 448)
    codes = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn)
    ref = codes.double().numpy() * scale
    assert np.array_equal(got, ref)
    assert np.all(got[3] == 0)
    # RNE bound: normal range relative error <= 2^-4; subnormal range absolute <= 2^-10 * scale
    err = np.abs(got / scale - y)
    normal = np.abs(y) >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(y[normal]) * 2.0 ** -4 + 1e-12)
    assert np.all(err[~normal] <= 2.0 ** -10 + 1e-15)
