"""Models of steps the e4m3-cache GPU path takes that the method itself does not.

NOT the oracle, and not a parity reference.  The fp8-cache decode multiplies
an e4m3 copy of the absorbed query (one scale per row) with the e4m3 cache;
that rounding is the kernel's choice, not part of what the method computes.
This module reproduces only that query rounding on top of the oracle's own
absorbed form, so that a test can separate the kernel's arithmetic error from
the error of the query quantisation.  Parity tests always compare with the
exact oracle (``oracle.mla_decode_expanded``); this model serves only as an
extra kernel-only check where the query rounding alone is larger than the
fp8 tolerance (sharp softmaxes).
"""

import numpy as np

import oracle

E4M3_MAX = 448.0


def quantize_rows_e4m3(x):
    """Each row of x as OCP e4m3 codes times one per-row scale, decoded back.

    The scale is the smallest power of two 2^k with max|row| / 2^k <= 448, so
    the row's largest magnitude lands in (224, 448] (1 for an all-zero row);
    codes are rounded to nearest-even by the oracle's codec.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    mant, ex = np.frexp(np.where(amax > 0, amax / E4M3_MAX, 1.0))
    ex = np.where(mant == 0.5, ex - 1, ex)
    scale = np.where(amax > 0, np.ldexp(1.0, np.clip(ex, -126, 127)), 1.0)
    return oracle.e4m3_bits_to_f64(oracle.f64_to_e4m3_bits(x / scale)) * scale


def decode_with_e4m3_query(inputs, rows):
    """The oracle's absorbed decode with q~ replaced by its per-row e4m3 form.

    Returns (q_latent, o_latent, out, lse) on the selected (b, j, h) rows.
    """
    q_nope, w_uk, w_uv = inputs["q_nope"], inputs["w_uk"], inputs["w_uv"]
    page, scale = int(inputs["page_size"]), float(inputs["softmax_scale"])
    q_len = q_nope.shape[1]
    n = len(rows)
    d_c, d_v = w_uk.shape[2], w_uv.shape[1]
    q_lat = np.zeros((n, d_c))
    o_lat = np.zeros((n, d_c))
    out = np.zeros((n, d_v))
    lse = np.full(n, -np.inf)
    for i, (b, j, h) in enumerate(np.asarray(rows)):
        b, j, h = int(b), int(j), int(h)
        length = int(inputs["seqlens"][b])
        c, kr = oracle.gather_cache(inputs["kv_latent"], inputs["kv_rope"],
                                    inputs["block_table"], b, length, page)
        pos = length - q_len + j
        n_vis = max(pos + 1 if inputs["causal"] else length, 0)
        q8 = quantize_rows_e4m3(w_uk[h].T @ q_nope[b, j, h])
        q_lat[i] = q8
        if n_vis == 0:
            continue
        qr = oracle.apply_rope(inputs["q_rope"][b, j, h], pos, inputs["rope_base"])
        s = scale * (c[:n_vis] @ q8 + kr[:n_vis] @ qr)
        m = s.max()
        e = np.exp(s - m)
        lse[i] = m + np.log(e.sum())
        o_lat[i] = (e / e.sum()) @ c[:n_vis]
        out[i] = w_uv[h] @ o_lat[i]
    return q_lat, o_lat, out, lse
