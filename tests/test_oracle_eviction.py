"""Pins for the eviction oracle (oracle/eviction.py).

The kept set is checked on hand-worked cases; the decode over it against the
full-cache oracle when nothing is evicted, against pure-Python brute force over
an explicit key list on tiny inputs, and on a planted needle: a key with a huge
score dominates the output when it is kept and changes nothing when it is
evicted.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.eviction import streaming_kept, mla_decode_streaming
from oracle_io import random_inputs


@pytest.mark.parametrize("length,sink,window,page,expect", [
    # window start 704 = floor((1000 - 256) / 64) * 64, past the 64 sinks
    (1000, 64, 256, 64, list(range(64)) + list(range(704, 1000))),
    # start 128 > 64 sinks
    (400, 64, 256, 64, list(range(64)) + list(range(128, 400))),
    # start 64 = the sinks' end: nothing to drop
    (321, 64, 256, 64, list(range(321))),
    # shorter than the window
    (200, 64, 256, 64, list(range(200))),
    # no sinks: the window alone (start floor((130 - 64) / 64) * 64 = 64)
    (130, 0, 64, 64, list(range(64, 130))),
    # page size 4: start floor((23 - 8) / 4) * 4 = 12
    (23, 4, 8, 4, [0, 1, 2, 3] + list(range(12, 23))),
    (0, 64, 256, 64, []),
])
def test_kept_sets(length, sink, window, page, expect):
    assert streaming_kept(length, sink, window, page).tolist() == expect


def _brute(inp, b, j, h, keys):
    """Attention of row (b, j, h) over the explicit key list (pure Python)."""
    page = inp["page_size"]
    L = int(inp["seqlens"][b])
    s_q = inp["q_nope"].shape[1]
    pos = L - s_q + j
    keys = [t for t in keys if (t <= pos or not inp["causal"])]
    if not keys:
        return None
    d = inp["q_rope"].shape[-1]
    qr_in = inp["q_rope"][b, j, h].tolist()
    qr = [0.0] * d
    for i in range(d // 2):
        th = inp["rope_base"] ** (-2.0 * i / d)
        c, s = math.cos(pos * th), math.sin(pos * th)
        qr[2 * i] = qr_in[2 * i] * c - qr_in[2 * i + 1] * s
        qr[2 * i + 1] = qr_in[2 * i] * s + qr_in[2 * i + 1] * c
    wuk, wuv = inp["w_uk"][h].tolist(), inp["w_uv"][h].tolist()
    qc = inp["q_nope"][b, j, h].tolist()
    d_c = len(wuk[0])
    sc, vs = [], []
    for t in keys:
        pg = int(inp["block_table"][b][t // page])
        c = inp["kv_latent"][pg][t % page].tolist()
        kr = inp["kv_rope"][pg][t % page].tolist()
        kc = [sum(wuk[n][e] * c[e] for e in range(d_c)) for n in range(len(wuk))]
        vs.append([sum(wuv[n][e] * c[e] for e in range(d_c)) for n in range(len(wuv))])
        sc.append(inp["softmax_scale"] * (sum(a * b_ for a, b_ in zip(qc, kc))
                                          + sum(a * b_ for a, b_ in zip(qr, kr))))
    m = max(sc)
    ex = [math.exp(x - m) for x in sc]
    tot = sum(ex)
    out = [sum(ex[t] / tot * vs[t][n] for t in range(len(keys))) for n in range(len(wuv))]
    return out, m + math.log(tot)


@pytest.mark.parametrize("q_len,causal", [(1, True), (2, True), (2, False)])
def test_streaming_decode_matches_brute_force(q_len, causal):
    rng = np.random.default_rng(40 + q_len)
    seqlens = [23, 9, 14, 3]
    inp = random_inputs(rng, batch=4, q_len=q_len, n_heads=2, d_c=4, d_rope=2, d_nope=3, d_v=5,
                        seqlens=seqlens, page_size=4, causal=causal, base=7.0)
    out, _, lse = mla_decode_streaming(inp, sink_tokens=4, window_tokens=8)
    i = 0
    for b in range(4):
        for j in range(q_len):
            for h in range(2):
                keys = streaming_kept(seqlens[b], 4, 8, 4).tolist()
                ref = _brute(inp, b, j, h, keys)
                if ref is None:
                    assert lse[i] == -np.inf
                else:
                    assert np.allclose(out[i], ref[0], rtol=1e-12, atol=1e-14)
                    assert abs(lse[i] - ref[1]) <= 1e-12 * max(1.0, abs(ref[1]))
                i += 1


def test_window_covering_everything_is_the_full_decode():
    rng = np.random.default_rng(44)
    inp = random_inputs(rng, batch=3, q_len=2, n_heads=3, d_c=8, d_rope=4, d_nope=6, d_v=5,
                        seqlens=[40, 17, 64], page_size=8)
    full = oracle.mla_decode_expanded(inp)
    out, o_lat, lse = mla_decode_streaming(inp, sink_tokens=8, window_tokens=64)
    assert np.allclose(out, full.out, rtol=1e-12, atol=1e-14)
    assert np.allclose(o_lat, full.o_latent, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, full.lse, rtol=1e-12)


@pytest.mark.parametrize("needle,kept", [(30, False), (2, True), (58, True)])
def test_needle_kept_or_evicted(needle, kept):
    """Token `needle` of a 60-token sequence gets a score far above the rest
    (its latent aligned with the query's absorbed direction).  With sinks
    0..7 and the window from token 48 on, it dominates when kept and is
    simply absent when evicted."""
    rng = np.random.default_rng(45)
    inp = random_inputs(rng, batch=1, q_len=1, n_heads=1, d_c=8, d_rope=2, d_nope=4, d_v=3,
                        seqlens=[60], page_size=8, causal=False)
    q_lat = inp["w_uk"][0].T @ inp["q_nope"][0, 0, 0]
    pg, sl = inp["block_table"][0][needle // 8], needle % 8
    inp["kv_latent"][pg, sl] = 200.0 * q_lat / np.linalg.norm(q_lat)
    assert streaming_kept(60, 8, 12, 8).tolist() == list(range(8)) + list(range(48, 60))
    out, _, _ = mla_decode_streaming(inp, sink_tokens=8, window_tokens=12)
    v_needle = inp["w_uv"][0] @ inp["kv_latent"][pg, sl]
    if kept:
        assert np.allclose(out[0], v_needle, rtol=1e-6, atol=1e-9)
    else:
        ref = _brute(inp, 0, 0, 0, list(range(8)) + list(range(48, 60)))
        assert np.allclose(out[0], ref[0], rtol=1e-12, atol=1e-14)
        assert not np.allclose(out[0], v_needle, rtol=1e-2)
