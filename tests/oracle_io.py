"""Turn a generated workload (storage form) into the oracle's fp64 inputs."""

import numpy as np

import oracle


def oracle_inputs(wl):
    return oracle.inputs_from_workload(wl)


def random_inputs(rng, batch, q_len, n_heads, d_c, d_rope, d_nope, d_v, seqlens,
                  page_size, shuffle=True, scale=None, base=10000.0, causal=True):
    """Small fp64 inputs drawn directly (for oracle self-tests)."""
    seqlens = np.asarray(seqlens)
    n_pages_seq = (seqlens + page_size - 1) // page_size
    needed = int(n_pages_seq.sum())
    num_pages = needed + 2
    perm = rng.permutation(num_pages) if shuffle else np.arange(num_pages)
    max_pages = max(1, int(n_pages_seq.max()))
    table = np.full((batch, max_pages), perm[-1], dtype=np.int64)
    off = 0
    for b in range(batch):
        k = int(n_pages_seq[b])
        table[b, :k] = perm[off:off + k]
        off += k
    return {
        "q_nope": rng.standard_normal((batch, q_len, n_heads, d_nope)),
        "q_rope": rng.standard_normal((batch, q_len, n_heads, d_rope)),
        "w_uk": rng.standard_normal((n_heads, d_nope, d_c)) / np.sqrt(d_c),
        "w_uv": rng.standard_normal((n_heads, d_v, d_c)) / np.sqrt(d_c),
        "kv_latent": rng.standard_normal((num_pages, page_size, d_c)),
        "kv_rope": rng.standard_normal((num_pages, page_size, d_rope)),
        "block_table": table,
        "seqlens": seqlens,
        "page_size": page_size,
        "softmax_scale": (1.0 / np.sqrt(d_nope + d_rope)) if scale is None else scale,
        "rope_base": base,
        "causal": causal,
    }
