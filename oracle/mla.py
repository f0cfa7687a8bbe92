"""fp64 reference for one MLA attention layer at decode time (test infrastructure only).

What the pages fix, and how this file writes it out:

* The cache holds, per token, only the compressed latent c_t^KV (d_c values)
  and the decoupled rotary key k_t^R (d_h^R values) ([LRKV] "Empirical Gains",
  the paragraph on what MLA caches, and FAQ "What does MLA store in the KV cache
  per token?").
* Content keys and values come from the latent through the up-projections:
  k^C_{t,i} = W^UK_i c_t and v_{t,i} = W^UV_i c_t ([LRKV] "Empirical Gains",
  the paragraph on absorbing W^UK and W^UV; [LKVC] "Core Concepts").
* Query and key each have a content part and a rotary part, concatenated
  before multi-head attention ([LKVC] "Operation Flow", steps 2-3).  Only the
  rotary parts are rotated ([LRKV] "Empirical Gains", decoupled RoPE).
* Attention itself is ordinary scaled dot-product attention over the cached
  tokens, one new query per step ([SLI] multi-head attention part and "Key
  Value Coverage").
* Absorbing W^UK into the query side and W^UV into the output side gives the
  same result and never materialises per-head K and V ([LRKV] "Empirical
  Gains" and FAQ "How does MLA optimize computation during inference?";
  [SNAP] two functionally equivalent kernel forms).

``mla_decode_expanded`` is the plain definition: gather the tokens through the
block table, expand K^C and V per head, run textbook masked softmax attention.
``mla_decode_absorbed`` is the absorbed form, kept only so tests can check the
equivalence above; it is never the reference for the GPU path.

Readings of points the pages leave open (softmax scale, rotary pairing and
frequencies, query position, causal rule for several query tokens, where V
comes from, empty rows) are listed in the design notes; the ones visible in
code are restated next to the code that takes them.
"""

from dataclasses import dataclass

import numpy as np

from .codecs import bf16_bits_to_f64, e4m3_bits_to_f64


def decode_stored(arr, dtype, scale=None):
    """Stored tensor -> float64.

    dtype 'f32' (float32 values), 'bf16' (uint16 bit patterns) or 'e4m3'
    (uint8 bit patterns, multiplied by a per-token float32 ``scale`` whose shape
    is ``arr.shape[:-1]``).
    """
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "e4m3":
        v = e4m3_bits_to_f64(arr)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return v * s[..., None]
    raise ValueError(f"unknown stored dtype {dtype!r}")


def rope_theta(d_rope, base):
    """Per-pair frequencies theta_i = base^(-2i/d_rope), i = 0 .. d_rope/2 - 1.

    The rotary page ([SLI] rotary-embedding part) rotates pair i of a vector at
    position p by the angle p * theta; its toy uses a single base frequency.
    The geometric frequency ladder with base 10000 is the reading taken here.
    """
    i = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / float(d_rope))


def apply_rope(x, pos, base):
    """Rotate the adjacent pairs (x_{2i}, x_{2i+1}) of ``x`` by pos * theta_i.

    Adjacent pairing follows the toy on the rotary page ([SLI]: the first two
    coordinates form one pair, the next two the next).  The rotation is the
    counter-clockwise 2-D rotation
        (a, b) -> (a cos - b sin, a sin + b cos).
    ``x`` has the rotary dimension last; ``pos`` broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def gather_cache(kv_latent, kv_rope, block_table, b, length, page_size):
    """Logical tokens 0..length-1 of sequence b through the block table.

    Token t lives in physical page block_table[b, t // page_size] at slot
    t % page_size.  Returns (C [length, d_c], KR [length, d_R]) in fp64.
    """
    t = np.arange(length)
    pages = np.asarray(block_table)[b, t // page_size]
    slots = t % page_size
    return kv_latent[pages, slots, :], kv_rope[pages, slots, :]


def expand_kv(c, w_uk_h, w_uv_h):
    """Per-head content keys and values from the latent: K^C = c W_UK^T, V = c W_UV^T.

    ``w_uk_h`` is [d_nope, d_c] and ``w_uv_h`` is [d_v, d_c] (each row maps the
    latent to one output coordinate).
    """
    return c @ w_uk_h.T, c @ w_uv_h.T


@dataclass
class DecodeResult:
    """Per selected row (b, j, h): everything the three library calls produce."""
    rows: np.ndarray       # [n, 3] int (b, j, h)
    q_latent: np.ndarray   # [n, d_c]   absorbed query q~
    q_pe: np.ndarray       # [n, d_R]   rotated rotary query
    o_latent: np.ndarray   # [n, d_c]   sum_t p_t c_t
    out: np.ndarray        # [n, d_v]   sum_t p_t v_t
    lse: np.ndarray        # [n]        natural-log log-sum-exp of the scores
    n_visible: np.ndarray  # [n]        number of keys the row attends to
    probs: list            # per row, the softmax weights (only if requested)


def _all_rows(batch, q_len, n_heads):
    b, j, h = np.meshgrid(np.arange(batch), np.arange(q_len), np.arange(n_heads),
                          indexing="ij")
    return np.stack([b.ravel(), j.ravel(), h.ravel()], axis=1)


def _visible(length, q_len, j, causal):
    """Keys a query row attends to.

    The new tokens are already in the cache, so query j of q_len sits at
    position pos_j = length - q_len + j.  With the causal rule it sees keys
    0..pos_j; without it, all ``length`` keys.  Returns (pos_j, n_visible);
    n_visible is clipped at 0 for rows with no key.
    """
    pos = length - q_len + j
    n_vis = pos + 1 if causal else length
    return pos, max(int(n_vis), 0)


def _decode(inputs, rows, return_probs, absorbed):
    q_nope = inputs["q_nope"]
    q_rope = inputs["q_rope"]
    w_uk = inputs["w_uk"]
    w_uv = inputs["w_uv"]
    kv_latent = inputs["kv_latent"]
    kv_rope = inputs["kv_rope"]
    block_table = np.asarray(inputs["block_table"])
    seqlens = np.asarray(inputs["seqlens"])
    page = int(inputs["page_size"])
    scale = float(inputs["softmax_scale"])
    base = float(inputs["rope_base"])
    causal = bool(inputs["causal"])
    batch, q_len, n_heads, _ = q_nope.shape
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    d_r = q_rope.shape[-1]

    rows = _all_rows(batch, q_len, n_heads) if rows is None else np.asarray(rows)
    n = len(rows)
    res = DecodeResult(rows=rows, q_latent=np.zeros((n, d_c)),
                       q_pe=np.zeros((n, d_r)), o_latent=np.zeros((n, d_c)),
                       out=np.zeros((n, d_v)), lse=np.full(n, -np.inf),
                       n_visible=np.zeros(n, dtype=np.int64), probs=[])
    # rows are visited in (b, h, j) order, so that the gathered cache of the
    # current sequence and the expansion of the current (sequence, head) serve
    # every row that shares them; results land at the rows' own positions
    gathered = {}
    expanded = {}
    probs = [None] * n
    order = np.lexsort((rows[:, 1], rows[:, 2], rows[:, 0])) if n else []
    for i in order:
        b, j, h = (int(x) for x in rows[i])
        length = int(seqlens[b])
        if b not in gathered:
            gathered = {b: gather_cache(kv_latent, kv_rope, block_table, b,
                                        length, page)}
            expanded = {}
        c, kr = gathered[b]
        pos, n_vis = _visible(length, q_len, j, causal)
        qc = q_nope[b, j, h]
        qr = apply_rope(q_rope[b, j, h], pos, base)
        q_lat = w_uk[h].T @ qc
        res.q_latent[i] = q_lat
        res.q_pe[i] = qr
        res.n_visible[i] = n_vis
        if n_vis == 0:
            probs[i] = np.zeros(0)
            continue
        if absorbed:
            s = scale * (c[:n_vis] @ q_lat + kr[:n_vis] @ qr)
        else:
            if h not in expanded:
                expanded = {h: expand_kv(c, w_uk[h], w_uv[h])}
            k_c, v = expanded[h]
            s = scale * (k_c[:n_vis] @ qc + kr[:n_vis] @ qr)
        m = np.max(s)
        e = np.exp(s - m)
        l_sum = np.sum(e)
        p = e / l_sum
        res.lse[i] = m + np.log(l_sum)
        res.o_latent[i] = p @ c[:n_vis]
        if absorbed:
            res.out[i] = w_uv[h] @ res.o_latent[i]
        else:
            res.out[i] = p @ v[:n_vis]
        probs[i] = p
    if return_probs:
        res.probs = probs
    return res


def mla_decode_expanded(inputs, rows=None, return_probs=False):
    """Plain definition: expand per-head K^C and V, then masked softmax attention.

    ``inputs`` is a dict of float64 arrays (already decoded):
      q_nope [B, s_q, H, d_nope], q_rope [B, s_q, H, d_R] (not yet rotated),
      w_uk [H, d_nope, d_c], w_uv [H, d_v, d_c],
      kv_latent [P, page, d_c] (dequantised), kv_rope [P, page, d_R] (stored
      already rotated at each token's own position),
      block_table [B, max_pages] int, seqlens [B] int,
    and scalars page_size, softmax_scale, rope_base, causal.
    ``rows`` selects (b, j, h) triples; default all, in (b, j, h) order.

    Score of key t for row (b, j, h):
      s_t = scale * ( q^C . (W_UK[h] c_t) + R(pos_j) q^R . k^R_t ),
    softmax over the visible keys, o = sum_t p_t W_UV[h] c_t.
    """
    return _decode(inputs, rows, return_probs, absorbed=False)


def mla_decode_absorbed(inputs, rows=None, return_probs=False):
    """Absorbed form: s_t = scale * (q~ . c_t + q_pe . k^R_t), o = W_UV[h] (sum_t p_t c_t).

    Kept only to check that absorption is exact ([LRKV] "Empirical Gains";
    [SNAP]): the tests pin it against the expanded form on the same inputs.
    """
    return _decode(inputs, rows, return_probs, absorbed=True)


def inputs_from_workload(wl):
    """Decode a generated workload's stored arrays into this module's fp64 inputs.

    ``wl`` is any object with the generator's fields (spec, kv_latent,
    kv_scale, kv_rope, q_nope, q_rope, w_uk, w_uv, block_table, seqlens); the
    oracle reads only those stored bits, through its own codecs.  Pinned
    field by field on a hand-built workload whose every array holds a
    different known code (tests/test_oracle_cache_and_inputs.py).
    """
    s = wl.spec
    return {
        "q_nope": decode_stored(wl.q_nope, s.act_dtype),
        "q_rope": decode_stored(wl.q_rope, s.act_dtype),
        "w_uk": decode_stored(wl.w_uk, s.act_dtype),
        "w_uv": decode_stored(wl.w_uv, s.act_dtype),
        "kv_latent": decode_stored(wl.kv_latent, s.latent_dtype, wl.kv_scale),
        "kv_rope": decode_stored(wl.kv_rope, s.act_dtype),
        "block_table": np.asarray(wl.block_table),
        "seqlens": np.asarray(wl.seqlens),
        "page_size": s.page_size,
        "softmax_scale": s.scale(),
        "rope_base": s.rope_base,
        "causal": s.causal,
    }
