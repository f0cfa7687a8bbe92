"""fp64 reference for decode over an evicted (bounded) latent cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports it.

The related-papers page ("Related papers: SnapMLA: Efficient Long-Context MLA
Decoding via H…", scifaro.com) names eviction techniques, StreamingLLM and
SnapKV among them, that keep a long context's KV cache bounded.  Its abstracts
are cut short, so the policy is a reading, listed with the design notes:

* Each sequence keeps its first ``sink_tokens`` tokens (the attention sinks)
  and its most recent tokens from the start of the page that holds token
  ``length - window_tokens`` on; every other token is dropped.  A sequence
  whose window would reach back into its sinks keeps everything.
* Kept keys stay at the positions they were cached at (their rotary part is
  stored already rotated), and each query keeps its true position, so a kept
  token's score is exactly its score in the full cache.
* With several query tokens the causal rule still applies: query j sees the
  kept keys at positions up to its own.

``mla_decode_streaming`` is then the plain definition: the expanded decode's
scores, restricted to the kept keys, under an ordinary softmax.

Pins (tests/test_oracle_eviction.py): hand-worked kept sets; a window that
covers the whole sequence reproduces ``mla_decode_expanded``; brute force
(pure-Python loops over an explicit key list) on tiny inputs; an evicted key
with a huge score changes nothing, a kept one dominates.
"""

import numpy as np

from .mla import apply_rope, gather_cache, expand_kv


def streaming_kept(length, sink_tokens, window_tokens, page_size):
    """Sorted indices of the tokens a sequence of ``length`` tokens keeps.

    The window starts at the page boundary at or below ``length -
    window_tokens``; when that start is not past the sinks, all tokens stay.
    """
    length = int(length)
    if length <= window_tokens:
        return np.arange(length)
    start = ((length - window_tokens) // page_size) * page_size
    if start <= sink_tokens:
        return np.arange(length)
    return np.concatenate([np.arange(sink_tokens), np.arange(start, length)])


def mla_decode_streaming(inputs, sink_tokens, window_tokens, rows=None):
    """Expanded decode over the kept keys only (``inputs`` as for
    ``mla_decode_expanded``).

    Returns (out [n, d_v], o_latent [n, d_c], lse [n]) for the selected
    (b, j, h) rows (default: all, in (b, j, h) order).
    """
    q_nope, q_rope = inputs["q_nope"], inputs["q_rope"]
    w_uk, w_uv = inputs["w_uk"], inputs["w_uv"]
    seqlens = np.asarray(inputs["seqlens"])
    page = int(inputs["page_size"])
    scale = float(inputs["softmax_scale"])
    base = float(inputs["rope_base"])
    causal = bool(inputs["causal"])
    batch, q_len, n_heads, _ = q_nope.shape
    if rows is None:
        b_, j_, h_ = np.meshgrid(np.arange(batch), np.arange(q_len), np.arange(n_heads),
                                 indexing="ij")
        rows = np.stack([b_.ravel(), j_.ravel(), h_.ravel()], axis=1)
    rows = np.asarray(rows)
    n = len(rows)
    d_c, d_v = w_uk.shape[2], w_uv.shape[1]
    out = np.zeros((n, d_v))
    o_lat = np.zeros((n, d_c))
    lse = np.full(n, -np.inf)
    gathered = {}
    for i, (b, j, h) in enumerate(rows):
        b, j, h = int(b), int(j), int(h)
        length = int(seqlens[b])
        if b not in gathered:
            # (one sequence's cache at a time)
            gathered = {b: gather_cache(inputs["kv_latent"], inputs["kv_rope"],
                                        inputs["block_table"], b, length, page)}
        c, kr = gathered[b]
        pos = length - q_len + j
        kept = streaming_kept(length, sink_tokens, window_tokens, page)
        if causal:
            kept = kept[kept <= pos]
        if kept.size == 0:
            continue
        k_c, v = expand_kv(c[kept], w_uk[h], w_uv[h])
        qr = apply_rope(q_rope[b, j, h], pos, base)
        s = scale * (k_c @ q_nope[b, j, h] + kr[kept] @ qr)
        m = np.max(s)
        e = np.exp(s - m)
        p = e / np.sum(e)
        lse[i] = m + np.log(np.sum(e))
        o_lat[i] = p @ c[kept]
        out[i] = p @ v
    return out, o_lat, lse
