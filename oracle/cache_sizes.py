"""Per-token KV-cache sizes, in elements (test infrastructure only).

[LRKV] "Empirical Gains: KV Footprint Reduction and Serving Speedups in
Practice" gives the per-token cache of each attention variant for l layers:
multi-head attention keeps 2 n_h d_h l, grouped-query attention 2 n_g d_h l,
multi-query attention 2 d_h l, and MLA (d_c + d_h^R) l; at the DeepSeek-V2
shape (n_h = 128, d_h = 128, d_c = 4 d_h, d_h^R = d_h / 2) the MLA figure is
4.5 d_h l, the same as grouped-query attention with 2.25 groups.

The model-level 93.3 % cache reduction and the 5.76x throughput figure on the
same page compare against another model whose configuration the pages do not
give; they are context only and nothing here computes them.
"""


def mla_cache_elems_per_token(d_c, d_rope, layers=1):
    return (d_c + d_rope) * layers


def mha_cache_elems_per_token(n_heads, d_head, layers=1):
    return 2 * n_heads * d_head * layers


def gqa_cache_elems_per_token(n_groups, d_head, layers=1):
    return 2 * n_groups * d_head * layers


def mqa_cache_elems_per_token(d_head, layers=1):
    return 2 * d_head * layers


def gqa_equivalent_groups(d_c, d_rope, d_head):
    """Number of GQA groups whose cache equals MLA's: (d_c + d_R) / (2 d_h)."""
    return (d_c + d_rope) / (2.0 * d_head)
