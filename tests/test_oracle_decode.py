"""Pins for the oracle's MLA decode.

Each test fixes the oracle against something other than itself: pure-Python
brute force on tiny shapes, torch's scaled_dot_product_attention (fp64, CPU)
as a library routine, the exact equivalence of absorbed and expanded attention
("Multi-Head Latent Attention: Scaling LLM Serving Throughput via Low-Rank KV
Compression", section "Empirical Gains", paragraph on absorbing W^UK/W^UV),
softmax definitions and special cases.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle_io import random_inputs


# ----------------------------------------------------------------------------
# pure-Python brute force (no numpy inside the arithmetic)

def _bf_rope(x, pos, base):
    d = len(x)
    out = [0.0] * d
    for i in range(d // 2):
        th = base ** (-2.0 * i / d)
        a, b = x[2 * i], x[2 * i + 1]
        c, s = math.cos(pos * th), math.sin(pos * th)
        out[2 * i] = a * c - b * s
        out[2 * i + 1] = a * s + b * c
    return out


def brute_force(inp, b, j, h):
    page = inp["page_size"]
    L = int(inp["seqlens"][b])
    s_q = inp["q_nope"].shape[1]
    pos = L - s_q + j
    n_vis = pos + 1 if inp["causal"] else L
    wuk = inp["w_uk"][h].tolist()          # [d_nope][d_c]
    wuv = inp["w_uv"][h].tolist()          # [d_v][d_c]
    qc = inp["q_nope"][b, j, h].tolist()
    qr = _bf_rope(inp["q_rope"][b, j, h].tolist(), pos, inp["rope_base"])
    d_c = len(wuk[0])
    scores, cs, vs = [], [], []
    for t in range(n_vis):
        pg = int(inp["block_table"][b][t // page])
        c = inp["kv_latent"][pg][t % page].tolist()
        kr = inp["kv_rope"][pg][t % page].tolist()
        k_c = [sum(wuk[n][e] * c[e] for e in range(d_c)) for n in range(len(wuk))]
        v = [sum(wuv[n][e] * c[e] for e in range(d_c)) for n in range(len(wuv))]
        sc = sum(qc[n] * k_c[n] for n in range(len(qc))) + sum(qr[i] * kr[i] for i in range(len(qr)))
        scores.append(inp["softmax_scale"] * sc)
        cs.append(c)
        vs.append(v)
    m = max(scores)
    ex = [math.exp(s - m) for s in scores]
    tot = sum(ex)
    p = [e / tot for e in ex]
    o = [sum(p[t] * vs[t][n] for t in range(n_vis)) for n in range(len(wuv))]
    ol = [sum(p[t] * cs[t][e] for t in range(n_vis)) for e in range(d_c)]
    lse = m + math.log(tot)
    qlat = [sum(wuk[n][e] * qc[n] for n in range(len(qc))) for e in range(d_c)]
    return o, ol, lse, qlat, qr, p


@pytest.mark.parametrize("q_len,seqlens,causal", [
    (1, [1, 5, 3], True), (2, [2, 5, 4], True), (2, [3, 5, 2], False), (1, [4], False)])
def test_oracle_matches_brute_force(q_len, seqlens, causal):
    rng = np.random.default_rng(10 + q_len + len(seqlens))
    inp = random_inputs(rng, batch=len(seqlens), q_len=q_len, n_heads=2, d_c=4,
                        d_rope=2, d_nope=3, d_v=5, seqlens=seqlens, page_size=2,
                        causal=causal, base=7.0)
    res = oracle.mla_decode_expanded(inp, return_probs=True)
    for i, (b, j, h) in enumerate(res.rows):
        o, ol, lse, qlat, qr, p = brute_force(inp, b, j, h)
        assert np.allclose(res.out[i], o, rtol=1e-12, atol=1e-14)
        assert np.allclose(res.o_latent[i], ol, rtol=1e-12, atol=1e-14)
        assert abs(res.lse[i] - lse) <= 1e-12 * max(1, abs(lse))
        assert np.allclose(res.q_latent[i], qlat, rtol=1e-12, atol=1e-14)
        assert np.allclose(res.q_pe[i], qr, rtol=1e-12, atol=1e-14)
        assert np.allclose(res.probs[i], p, rtol=1e-12, atol=1e-15)


def _sdpa_reference(inp, b, j, h):
    """torch SDPA (fp64, CPU) on explicitly expanded [q^C; R q^R] and [K^C; k^R]."""
    page = inp["page_size"]
    L = int(inp["seqlens"][b])
    s_q = inp["q_nope"].shape[1]
    pos = L - s_q + j
    n_vis = pos + 1 if inp["causal"] else L
    t = np.arange(L)
    pages = inp["block_table"][b, t // page]
    c = inp["kv_latent"][pages, t % page]
    kr = inp["kv_rope"][pages, t % page]
    k = np.concatenate([c @ inp["w_uk"][h].T, kr], axis=1)
    v = c @ inp["w_uv"][h].T
    ang = pos * inp["rope_base"] ** (-2.0 * np.arange(kr.shape[1] // 2) / kr.shape[1])
    qr = inp["q_rope"][b, j, h].copy()
    rot = np.empty_like(qr)
    rot[0::2] = qr[0::2] * np.cos(ang) - qr[1::2] * np.sin(ang)
    rot[1::2] = qr[0::2] * np.sin(ang) + qr[1::2] * np.cos(ang)
    q = np.concatenate([inp["q_nope"][b, j, h], rot])
    mask = torch.from_numpy(t < n_vis)[None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], attn_mask=mask, scale=inp["softmax_scale"])
    return out[0, 0].numpy()


def test_oracle_matches_torch_sdpa():
    rng = np.random.default_rng(11)
    inp = random_inputs(rng, batch=3, q_len=2, n_heads=4, d_c=32, d_rope=8,
                        d_nope=16, d_v=12, seqlens=[70, 129, 2], page_size=16)
    res = oracle.mla_decode_expanded(inp)
    for i, (b, j, h) in enumerate(res.rows):
        ref = _sdpa_reference(inp, b, j, h)
        assert np.allclose(res.out[i], ref, rtol=1e-10, atol=1e-12)


def test_absorbed_equals_expanded():
    rng = np.random.default_rng(12)
    inp = random_inputs(rng, batch=2, q_len=2, n_heads=8, d_c=64, d_rope=16,
                        d_nope=32, d_v=32, seqlens=[300, 77], page_size=64)
    a = oracle.mla_decode_absorbed(inp)
    e = oracle.mla_decode_expanded(inp)
    for x, y in [(a.out, e.out), (a.o_latent, e.o_latent), (a.lse, e.lse)]:
        assert np.max(np.abs(x - y)) <= 1e-12 * np.max(np.abs(y))


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(13)
    inp = random_inputs(rng, batch=2, q_len=2, n_heads=3, d_c=16, d_rope=4,
                        d_nope=8, d_v=8, seqlens=[50, 9], page_size=8)
    res = oracle.mla_decode_expanded(inp, return_probs=True)
    for i, p in enumerate(res.probs):
        assert len(p) == res.n_visible[i]
        assert abs(p.sum() - 1.0) <= 1e-14
        assert np.all(p >= 0)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(14)
    inp = random_inputs(rng, batch=2, q_len=1, n_heads=3, d_c=16, d_rope=4,
                        d_nope=8, d_v=8, seqlens=[1, 1], page_size=8)
    res = oracle.mla_decode_expanded(inp)
    for i, (b, j, h) in enumerate(res.rows):
        pg = inp["block_table"][b, 0]
        c0 = inp["kv_latent"][pg, 0]
        assert np.allclose(res.o_latent[i], c0, rtol=1e-15, atol=0)
        assert np.allclose(res.out[i], inp["w_uv"][h] @ c0, rtol=1e-13)


def test_zero_query_gives_mean_latent():
    rng = np.random.default_rng(15)
    inp = random_inputs(rng, batch=2, q_len=2, n_heads=2, d_c=16, d_rope=4,
                        d_nope=8, d_v=8, seqlens=[40, 13], page_size=8)
    inp["q_nope"][:] = 0
    inp["q_rope"][:] = 0
    res = oracle.mla_decode_expanded(inp)
    for i, (b, j, h) in enumerate(res.rows):
        n = res.n_visible[i]
        t = np.arange(n)
        pages = inp["block_table"][b, t // 8]
        mean = inp["kv_latent"][pages, t % 8].mean(axis=0)
        assert np.allclose(res.o_latent[i], mean, rtol=1e-13, atol=1e-15)
        assert abs(res.lse[i] - math.log(n)) <= 1e-13


def test_mtp_first_token_equals_single_token_at_shorter_length():
    """With two causal query tokens, token 0 at length L sees what a single query at L-1 sees."""
    rng = np.random.default_rng(16)
    inp2 = random_inputs(rng, batch=2, q_len=2, n_heads=4, d_c=32, d_rope=8,
                         d_nope=16, d_v=16, seqlens=[65, 130], page_size=16)
    inp1 = dict(inp2)
    inp1["q_nope"] = inp2["q_nope"][:, :1].copy()
    inp1["q_rope"] = inp2["q_rope"][:, :1].copy()
    inp1["seqlens"] = inp2["seqlens"] - 1
    r2 = oracle.mla_decode_expanded(inp2)
    r1 = oracle.mla_decode_expanded(inp1)
    sel = r2.rows[:, 1] == 0
    assert np.allclose(r2.out[sel], r1.out, rtol=1e-13, atol=1e-15)
    assert np.allclose(r2.lse[sel], r1.lse, rtol=1e-13)
    # and token 1 attends to one more key than token 0
    assert np.all(r2.n_visible[r2.rows[:, 1] == 1] == r2.n_visible[sel] + 1)


def test_block_table_permutation_is_invisible():
    rng = np.random.default_rng(17)
    inp = random_inputs(rng, batch=2, q_len=1, n_heads=2, d_c=8, d_rope=4,
                        d_nope=4, d_v=4, seqlens=[33, 20], page_size=4, shuffle=False)
    ref = oracle.mla_decode_expanded(inp)
    perm = rng.permutation(inp["kv_latent"].shape[0])
    inv = np.argsort(perm)
    moved = dict(inp)
    moved["kv_latent"] = inp["kv_latent"][perm]
    moved["kv_rope"] = inp["kv_rope"][perm]
    moved["block_table"] = inv[inp["block_table"]]
    got = oracle.mla_decode_expanded(moved)
    assert np.array_equal(got.out, ref.out)
    assert np.array_equal(got.lse, ref.lse)


def test_row_with_no_visible_key():
    rng = np.random.default_rng(18)
    inp = random_inputs(rng, batch=1, q_len=2, n_heads=2, d_c=8, d_rope=4,
                        d_nope=4, d_v=4, seqlens=[1], page_size=4)
    res = oracle.mla_decode_expanded(inp)
    for i, (b, j, h) in enumerate(res.rows):
        if j == 0:                      # position -1: nothing to attend to
            assert res.n_visible[i] == 0
            assert np.all(res.out[i] == 0) and res.lse[i] == -np.inf
        else:
            assert res.n_visible[i] == 1


def test_row_subset_matches_full_run():
    rng = np.random.default_rng(19)
    inp = random_inputs(rng, batch=3, q_len=2, n_heads=4, d_c=16, d_rope=4,
                        d_nope=8, d_v=8, seqlens=[21, 40, 5], page_size=8)
    full = oracle.mla_decode_expanded(inp)
    pick = np.array([[2, 1, 3], [0, 0, 0], [1, 1, 2]])
    sub = oracle.mla_decode_expanded(inp, rows=pick)
    for i, (b, j, h) in enumerate(pick):
        k = (b * 2 + j) * 4 + h
        assert np.array_equal(sub.out[i], full.out[k])
        assert np.array_equal(sub.o_latent[i], full.o_latent[k])


def test_e4m3_query_kernel_model():
    """The kernel model of tests/kernel_models.py (the per-row e4m3 query of the
    fp8-cache path) equals the exact oracle when every absorbed query row is
    already an e4m3 code times its scale (W_UK[h] the identity, q^C drawn from
    e4m3 codes with the row maximum at 448 * 2^-4), and moves the result when
    the query is not representable."""
    import kernel_models
    rng = np.random.default_rng(41)
    d = 16
    inp = random_inputs(rng, batch=2, q_len=2, n_heads=3, d_c=d, d_rope=8, d_nope=d,
                        d_v=16, seqlens=[70, 9], page_size=16)
    codes = rng.integers(0, 0x7F, size=inp["q_nope"].shape)      # finite e4m3 codes
    q = oracle.e4m3_bits_to_f64(codes.astype(np.uint8)) * 2.0 ** -4
    q[..., 0] = 448.0 * 2.0 ** -4                                   # each row's maximum
    inp["q_nope"] = q
    inp["w_uk"] = np.broadcast_to(np.eye(d), (3, d, d)).copy()
    rows = oracle.mla_decode_expanded(inp).rows
    exact = oracle.mla_decode_expanded(inp, rows=rows)
    q_lat, o_lat, out, lse = kernel_models.decode_with_e4m3_query(inp, rows)
    assert np.array_equal(q_lat, exact.q_latent)
    assert np.allclose(o_lat, exact.o_latent, rtol=1e-12, atol=1e-14)
    assert np.allclose(out, exact.out, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse[np.isfinite(lse)], exact.lse[np.isfinite(exact.lse)], rtol=1e-12)
    # a general query is rounded: the model's result moves away from the oracle's
    inp2 = random_inputs(rng, batch=2, q_len=2, n_heads=3, d_c=32, d_rope=8, d_nope=16,
                         d_v=16, seqlens=[70, 9], page_size=16)
    ex2 = oracle.mla_decode_expanded(inp2)
    _, o2, _, _ = kernel_models.decode_with_e4m3_query(inp2, ex2.rows)
    assert not np.allclose(o2, ex2.o_latent, rtol=1e-6, atol=0)
