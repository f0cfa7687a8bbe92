"""Pins of oracle/projections.py: pure-Python loops on tiny shapes, and the
pages' absorption identity on a whole decode step (absorbed weights give the
same layer output as applying W^UQ, W^UK, W^UV and W^O one at a time)."""

import numpy as np
import pytest

import oracle
from oracle_io import random_inputs


def _loops_matmul_rows(h, w):
    T, D = len(h), len(h[0])
    O = len(w)
    return [[sum(w[o][d] * h[t][d] for d in range(D)) for o in range(O)] for t in range(T)]


def test_down_project_brute_force():
    rng = np.random.default_rng(1)
    h, w = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    assert np.allclose(oracle.down_project(h, w), _loops_matmul_rows(h.tolist(), w.tolist()),
                       rtol=1e-13, atol=1e-13)


def test_up_project_query_brute_force():
    rng = np.random.default_rng(2)
    T, H, dn, dr, dq = 2, 3, 4, 2, 5
    c, wuq, wqr = (rng.standard_normal(s) for s in ((T, dq), (H, dn, dq), (H, dr, dq)))
    qn, qr = oracle.up_project_query(c, wuq, wqr)
    for t in range(T):
        for i in range(H):
            for n in range(dn):
                assert abs(qn[t, i, n] - sum(wuq[i, n, q] * c[t, q] for q in range(dq))) < 1e-12
            for r in range(dr):
                assert abs(qr[t, i, r] - sum(wqr[i, r, q] * c[t, q] for q in range(dq))) < 1e-12


def test_absorbed_query_weights_brute_force():
    """W~[i, c, q] = sum_n W_UK[i, n, c] W_UQ[i, n, q], looped out."""
    rng = np.random.default_rng(3)
    H, dn, dc, dq = 2, 3, 4, 5
    wuq, wuk = rng.standard_normal((H, dn, dq)), rng.standard_normal((H, dn, dc))
    got = oracle.absorb_query_weights(wuq, wuk)
    assert got.shape == (H, dc, dq)
    for i in range(H):
        for c in range(dc):
            for q in range(dq):
                ref = sum(wuk[i, n, c] * wuq[i, n, q] for n in range(dn))
                assert abs(got[i, c, q] - ref) < 1e-12


def test_absorbed_output_weights_brute_force():
    """W~O[m, i d_c + c] = sum_v W_O[m, i d_v + v] W_UV[i, v, c], looped out."""
    rng = np.random.default_rng(4)
    H, dv, dc, dm = 3, 2, 4, 5
    wo, wuv = rng.standard_normal((dm, H * dv)), rng.standard_normal((H, dv, dc))
    got = oracle.absorb_output_weights(wo, wuv)
    assert got.shape == (dm, H * dc)
    for m in range(dm):
        for i in range(H):
            for c in range(dc):
                ref = sum(wo[m, i * dv + v] * wuv[i, v, c] for v in range(dv))
                assert abs(got[m, i * dc + c] - ref) < 1e-12


@pytest.mark.parametrize("q_len", [1, 3])
def test_absorbed_weights_reproduce_the_layer(q_len):
    """A decode step from hidden states to the layer output, two ways:
    (1) q^C, q^R = W_UQ c^Q, W_QR c^Q; expanded attention (K^C = W_UK c, V = W_UV c);
        y = W_O [o_1; ...; o_H];
    (2) q~ = W~ c^Q with W~ = W_UK^T W_UQ (the absorbed query weights) equals the
        decode's absorbed query, and y = W~O [o~_1; ...; o~_H] with W~O = W_O W_UV."""
    rng = np.random.default_rng(10 + q_len)
    H, dn, dr, dc, dv, dq, dm = 3, 6, 4, 8, 5, 12, 16
    B = 2
    inp = random_inputs(rng, batch=B, q_len=q_len, n_heads=H, d_c=dc, d_rope=dr, d_nope=dn,
                        d_v=dv, seqlens=[9, 14], page_size=4)
    h = rng.standard_normal((B * q_len, dm))
    w_dq = rng.standard_normal((dq, dm)) / np.sqrt(dm)
    w_uq = rng.standard_normal((H, dn, dq)) / np.sqrt(dq)
    w_qr = rng.standard_normal((H, dr, dq)) / np.sqrt(dq)
    w_o = rng.standard_normal((dm, H * dv)) / np.sqrt(H * dv)
    c_q = oracle.down_project(h, w_dq)
    q_nope, q_rope = oracle.up_project_query(c_q, w_uq, w_qr)
    inp["q_nope"] = q_nope.reshape(B, q_len, H, dn)
    inp["q_rope"] = q_rope.reshape(B, q_len, H, dr)
    ref = oracle.mla_decode_expanded(inp)
    y1 = oracle.output_project(ref.out.reshape(B * q_len, H * dv), w_o)
    # (2) the absorbed weights
    w_qabs = oracle.absorb_query_weights(w_uq, inp["w_uk"])
    q_abs = np.einsum("hcq,tq->thc", w_qabs, c_q).reshape(B * q_len * H, dc)
    assert np.allclose(q_abs, ref.q_latent, rtol=1e-12, atol=1e-12)
    w_oabs = oracle.absorb_output_weights(w_o, inp["w_uv"])
    y2 = oracle.output_project(ref.o_latent.reshape(B * q_len, H * dc), w_oabs)
    assert np.allclose(y1, y2, rtol=1e-11, atol=1e-12)
    # heads paired with the wrong W_UQ, or output columns one head off, break it
    bad = oracle.absorb_query_weights(np.roll(w_uq, 1, axis=0), inp["w_uk"])
    q_bad = np.einsum("hcq,tq->thc", bad, c_q).reshape(B * q_len * H, dc)
    assert not np.allclose(q_bad, ref.q_latent, rtol=1e-6)
    shifted = np.roll(w_oabs, dc, axis=1)
    assert not np.allclose(oracle.output_project(ref.o_latent.reshape(B * q_len, H * dc),
                                                 shifted), y1, rtol=1e-6)
