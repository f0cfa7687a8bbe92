"""MLA (Multi-Head Latent Attention) decode over a paged latent KV cache, for
AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI declared in
include/mla_decode.h (libmla_decode.so, built in-tree by
``python -m head_latent_attention_03_amd.build``).  This package holds the
thin ctypes binding of that ABI (same function names), device-buffer
marshalling for a decode batch, and the seeded synthetic workloads.
"""

from ._binding import (LIBRARY_PATH, MLA_BF16, MLA_F32, MLA_FP8_E4M3, MlaDims, MlaError,
                       load_library, mla_absorb_q, mla_append_kv, mla_combine,
                       mla_decode_paged, mla_decode_workspace_size, mla_status_string)

__all__ = [
    "LIBRARY_PATH", "MLA_BF16", "MLA_F32", "MLA_FP8_E4M3", "MlaDims", "MlaError",
    "load_library", "mla_absorb_q", "mla_append_kv", "mla_combine", "mla_decode_paged",
    "mla_decode_workspace_size", "mla_status_string",
]
