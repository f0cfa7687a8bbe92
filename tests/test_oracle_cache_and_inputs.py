"""Cache-size closed forms printed on the pages, and properties of the input generator."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from head_latent_attention_03_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepseek_v2_cache.json")


def test_cache_closed_forms_match_the_page():
    g = json.load(open(GOLDEN))
    n_h, d_h, d_c, d_r = g["n_h"], g["d_h"], g["d_c"], g["d_h_R"]
    assert d_c == g["d_c_over_d_h"] * d_h and d_h == g["d_h_over_d_h_R"] * d_r
    mla = oracle.mla_cache_elems_per_token(d_c, d_r)
    assert mla == 576
    assert mla == g["mla_cache_over_d_h"] * d_h
    assert oracle.gqa_equivalent_groups(d_c, d_r, d_h) == g["gqa_equivalent_groups"]
    assert oracle.gqa_cache_elems_per_token(g["gqa_equivalent_groups"], d_h) == mla
    mha = oracle.mha_cache_elems_per_token(n_h, d_h)
    assert mha == 32768
    assert abs(mla / mha - 0.017578125) < 1e-15
    assert oracle.mqa_cache_elems_per_token(d_h) == 256
    # l layers scale every figure linearly
    assert oracle.mla_cache_elems_per_token(d_c, d_r, 60) == 60 * mla


@pytest.mark.parametrize("n,bytes_per_token", [(2, 1152), (4, 644)])
def test_cache_bytes_per_token(n, bytes_per_token):
    spec = inputs.workload(n, batch=2, seqlen=70)
    assert inputs.cache_bytes_per_token(spec) == bytes_per_token
    wl = inputs.make_workload(spec)
    per_tok = (wl.kv_latent[0, 0].nbytes + wl.kv_rope[0, 0].nbytes
               + (wl.kv_scale[0, 0].nbytes if wl.kv_scale is not None else 0))
    assert per_tok == bytes_per_token


def test_generator_is_seeded_and_poisons_unused_storage():
    spec = inputs.workload(2, batch=3, seqlen=[100, 64, 1])
    a = inputs.make_workload(spec)
    b = inputs.make_workload(spec)
    assert np.array_equal(a.kv_latent, b.kv_latent) and np.array_equal(a.q_nope, b.q_nope)
    lat = oracle.decode_stored(a.kv_latent, "bf16")
    used = set()
    for bi, L in enumerate(a.seqlens):
        n_p = (L + 63) // 64
        for k in range(a.block_table.shape[1]):
            p = a.block_table[bi, k]
            if k < n_p:
                used.add(int(p))
                lo = L - 64 * k
                assert np.all(np.isfinite(lat[p, :min(lo, 64)]))
                if lo < 64:
                    assert np.all(np.isnan(lat[p, lo:]))
            else:
                assert np.all(np.isnan(lat[p]))
    spare = [p for p in range(a.num_pages) if p not in used]
    assert len(spare) >= 1 and np.all(np.isnan(lat[spare]))
    assert len(used) == sum((L + 63) // 64 for L in a.seqlens)


def test_fp8_latent_scales():
    spec = inputs.workload(4, batch=2, seqlen=130)
    wl = inputs.make_workload(spec)
    deq = oracle.decode_stored(wl.kv_latent, "e4m3", wl.kv_scale)
    codes = oracle.e4m3_bits_to_f64(wl.kv_latent)
    p = wl.block_table[0, 0]
    # each token's largest code is the largest finite e4m3 value
    assert np.all(np.max(np.abs(codes[p]), axis=-1) == 448.0)
    assert np.all(np.isfinite(deq[p]))
    assert 1.5 < np.max(np.abs(deq[p])) < 8.0          # N(0,1) draws


def test_seqlen_rules():
    s3 = inputs.workload(3, batch=4096)
    L = inputs.draw_seqlens(s3, np.random.default_rng(0))
    assert L.min() >= 16384 and L.max() <= 65536
    s5 = inputs.workload(5, batch=200000)
    L = inputs.draw_seqlens(s5, np.random.default_rng(0))
    assert L.min() >= 2 and L.max() <= 32768
    # arithmetic mean 2048 before clipping (the cap removes a sliver of the tail)
    assert abs(L.mean() - 2048) < 40
    assert abs(np.median(L) - 2048 * math.exp(-0.5)) < 30


@pytest.mark.parametrize("latent_dtype", ["bf16", "e4m3"])
def test_inputs_from_workload_maps_every_field(latent_dtype):
    """inputs_from_workload on a hand-built workload: every stored array holds its
    own known code and has its own shape, so a swapped field (W_UK for W_UV, the
    rotary key for the latent), a wrong decoding or a lost scale shows up.
    Expected values come from the bf16 / e4m3 format definitions, written out:
    bf16 0x3F80 = 1, 0x4000 = 2, 0x4040 = 3, 0x4080 = 4, 0x40A0 = 5, 0x40C0 = 6;
    e4m3 0x40 = 2 (exponent 8 - 7, mantissa 0), times the token scale 0.25."""
    from types import SimpleNamespace
    B, S, H, d_c, d_r, d_n, d_v, P, page = 2, 3, 5, 16, 4, 6, 7, 3, 8
    spec = SimpleNamespace(act_dtype="bf16", latent_dtype=latent_dtype, page_size=page,
                           rope_base=1234.5, causal=False, scale=lambda: 0.375)
    full = lambda shape, code, dt=np.uint16: np.full(shape, code, dtype=dt)
    if latent_dtype == "bf16":
        kv_latent, kv_scale, lat_val = full((P, page, d_c), 0x40A0), None, 5.0
    else:
        kv_latent = full((P, page, d_c), 0x40, np.uint8)
        kv_scale = np.full((P, page), 0.25, dtype=np.float32)
        lat_val = 0.5
    table = np.array([[2, 0], [1, 2]], dtype=np.int32)
    wl = SimpleNamespace(spec=spec, q_nope=full((B, S, H, d_n), 0x3F80),
                         q_rope=full((B, S, H, d_r), 0x4000),
                         w_uk=full((H, d_n, d_c), 0x4040), w_uv=full((H, d_v, d_c), 0x4080),
                         kv_latent=kv_latent, kv_scale=kv_scale,
                         kv_rope=full((P, page, d_r), 0x40C0), block_table=table,
                         seqlens=np.array([9, 16], dtype=np.int32))
    got = oracle.inputs_from_workload(wl)
    expect = {"q_nope": ((B, S, H, d_n), 1.0), "q_rope": ((B, S, H, d_r), 2.0),
              "w_uk": ((H, d_n, d_c), 3.0), "w_uv": ((H, d_v, d_c), 4.0),
              "kv_latent": ((P, page, d_c), lat_val), "kv_rope": ((P, page, d_r), 6.0)}
    for name, (shape, val) in expect.items():
        assert got[name].shape == shape, name
        assert got[name].dtype == np.float64, name
        assert np.all(got[name] == val), name
    assert np.array_equal(got["block_table"], table)
    assert np.array_equal(got["seqlens"], [9, 16])
    assert got["page_size"] == page and got["softmax_scale"] == 0.375
    assert got["rope_base"] == 1234.5 and got["causal"] is False
    assert set(got) == set(expect) | {"block_table", "seqlens", "page_size", "softmax_scale",
                                      "rope_base", "causal"}
