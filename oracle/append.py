"""fp64 reference for appending new tokens to the paged latent cache (test
infrastructure only).

What a decode step writes into the cache for each new token, as the pages fix
it and as this file writes it out:

* The cache holds, per token, only the compressed latent c_t^KV and the
  decoupled rotary key k_t^R ([LRKV] "Empirical Gains", the paragraph on what
  MLA caches; [LKVC] "KV Cache Compression").
* The latent is normalised by RMSNorm, in FP32 ("FP8 Mixed-Precision
  Training", same tag page as [LKVC], section "Three Main Architectures",
  the Multi-head Latent Attention item: key/value compression in BF16, then
  RMSNorm in FP32 for stability).
* The rotary key carries the position: RoPE, in FP32 ([LKVC] "FP8/FP32 Mixed
  Precision"; "Operation Flow", step 5).  It is stored already rotated, so the
  decode rotates only the query.
* With an e4m3 cache the latent is quantised ([LKVC] "FP8/FP32 Mixed
  Precision": FP8 for the matrix products that consume it).

Readings of what the pages leave open (listed in the design notes):

* RMSNorm is y = x / sqrt(mean(x^2) + eps) * g with a per-coordinate gain g
  and eps = 1e-6 (the pages name RMSNorm but give neither the formula's eps
  nor the gain; this is the usual definition).
* A new token's position is seqlens[b] - q_len + j, the same rule the query
  side uses (the lengths already count the new tokens); a token whose position
  is negative is not written.
* The e4m3 latent is stored as codes of y / s with s = max|y| / 448 per token
  (1 for an all-zero row), rounded to nearest-even and saturated at +-448: the
  same per-token quantiser the synthetic fp8 caches use.

Pins (``tests/test_oracle_append.py``): RMSNorm closed forms (a constant
vector, the RMS of the output, scale invariance at eps = 0), a placement case
worked by hand, and the RoPE and e4m3 pins of the other oracle modules, which
this file reuses.
"""

import numpy as np

from .codecs import E4M3_MAX, f64_to_bf16_bits, f64_to_e4m3_bits
from .mla import apply_rope

RMS_EPS = 1e-6


def rms_norm(x, gain, eps=RMS_EPS):
    """y = x / sqrt(mean(x^2) + eps) * gain over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def append_positions(seqlens, q_len, block_table, page_size):
    """Where each new token (b, j) goes: (position, page, slot), position -1 and
    page / slot -1 for a token that is not written (negative position)."""
    seqlens = np.asarray(seqlens)
    table = np.asarray(block_table)
    B = len(seqlens)
    pos = np.full((B, q_len), -1, dtype=np.int64)
    page = np.full((B, q_len), -1, dtype=np.int64)
    slot = np.full((B, q_len), -1, dtype=np.int64)
    for b in range(B):
        for j in range(q_len):
            p = int(seqlens[b]) - q_len + j
            if p < 0:
                continue
            pos[b, j] = p
            page[b, j] = table[b, p // page_size]
            slot[b, j] = p % page_size
    return pos, page, slot


def quantize_token_e4m3(y):
    """One token's latent as (e4m3 codes, scale): s = max|y| / 448 (1 if y = 0),
    codes = nearest-even e4m3 of y / s, saturated at +-448."""
    y = np.asarray(y, dtype=np.float64)
    amax = np.max(np.abs(y), axis=-1, keepdims=True)
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return f64_to_e4m3_bits(y / s), s[..., 0]


def append_kv(kv_c, k_rope, gain, seqlens, q_len, block_table, page_size, rope_base,
              eps=RMS_EPS):
    """The cache writes of one step, in fp64.

    kv_c [B, q_len, d_c] (the latent before RMSNorm) and k_rope [B, q_len, d_R]
    (before RoPE) are decoded inputs.  Returns a dict with the placement
    (``pos``, ``page``, ``slot``, each [B, q_len]), the normalised latent ``y``
    [B, q_len, d_c] and the rotated key ``kr`` [B, q_len, d_R], plus their
    stored forms: ``y_bf16`` (bit patterns), ``y_e4m3`` (codes) with
    ``y_scale``, ``kr_bf16`` (bit patterns).
    """
    pos, page, slot = append_positions(seqlens, q_len, block_table, page_size)
    y = rms_norm(kv_c, gain, eps)
    kr = apply_rope(k_rope, np.maximum(pos, 0), rope_base)
    codes, scale = quantize_token_e4m3(y)
    return {
        "pos": pos, "page": page, "slot": slot,
        "y": y, "kr": kr,
        "y_bf16": f64_to_bf16_bits(y), "y_e4m3": codes, "y_scale": scale,
        "kr_bf16": f64_to_bf16_bits(kr),
    }
