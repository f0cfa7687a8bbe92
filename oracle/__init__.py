"""CPU oracle for MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never does,
and this package imports nothing from the product path.

Everything here is plain, slow and written to be checked by eye against the
pages it follows:

* [LRKV]  "Multi-Head Latent Attention: Scaling LLM Serving Throughput via
  Low-Rank KV Compression" (priorstack.com, tag page "Deep Learning
  Architecture"), sections "TL;DR", "The Memory Wall", "Empirical Gains: KV
  Footprint Reduction and Serving Speedups in Practice", "Closing thoughts",
  "Frequently Asked Questions".
* [LKVC]  "Multi-Head Latent Attention – Latent KV-Cache (DeepSeek v3)"
  (eeumee.net, tag page "MixedPrecision"), sections "Core Concepts",
  "Operation Flow", "FP8/FP32 Mixed Precision", "Residual & RoPE Explanation".
* [SLI]   "Deepseek-V3 Define 1: Higher Attachment of Head | by Shirley Li"
  (dataforcee.us), the multi-head-attention part, "Key Value Coverage" (the
  KV cache) and the rotary-embedding part ("Cords (rotating rotation").
* [LKVC] "Operation Flow" and [LRKV] "Empirical Gains" also fix the dense
  products around the attention (down-projections, query up-projection,
  weight-level absorption), in ``projections``.
* "FP8 Mixed-Precision Training" (eeumee.net, the same tag page as [LKVC]),
  section "Three Main Architectures" (RMSNorm of the compressed key/value in
  FP32), for the cache append.
* [SNAP]  "Related papers: SnapMLA: Efficient Long-Context MLA Decoding via H…"
  (scifaro.com), the abstract on two functionally equivalent kernel forms, and
  the abstracts naming cache-eviction techniques (StreamingLLM, SnapKV), for
  the decode over an evicted cache in ``eviction``.

Floating point is fp64 throughout.  Stored inputs (bf16 / OCP e4m3 bit
patterns) are decoded by this package's own codecs.

Parity status of each function is stated in its docstring; nothing here is
"parity unpinned" except the model-level figures quoted in ``cache_sizes``
(93.3 % and 5.76x), which are context only and are not computed.
"""

from .codecs import (bf16_bits_to_f64, f64_to_bf16_bits, e4m3_bits_to_f64,
                     f64_to_e4m3_bits, E4M3_MAX)
from .mla import (rope_theta, apply_rope, gather_cache, expand_kv,
                  mla_decode_expanded, mla_decode_absorbed,
                  decode_stored, DecodeResult, inputs_from_workload)
from .append import (rms_norm, append_positions, quantize_token_e4m3, append_kv,
                     RMS_EPS)
from .projections import (down_project, up_project_query, absorb_query_weights,
                          absorb_output_weights, output_project)
from .eviction import streaming_kept, mla_decode_streaming
from .cache_sizes import (mla_cache_elems_per_token, mha_cache_elems_per_token,
                          gqa_cache_elems_per_token, mqa_cache_elems_per_token,
                          gqa_equivalent_groups)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "e4m3_bits_to_f64",
    "f64_to_e4m3_bits", "E4M3_MAX", "rope_theta", "apply_rope", "gather_cache",
    "expand_kv", "mla_decode_expanded", "mla_decode_absorbed",
    "decode_stored", "DecodeResult", "inputs_from_workload",
    "rms_norm", "append_positions", "quantize_token_e4m3", "append_kv", "RMS_EPS",
    "down_project", "up_project_query", "absorb_query_weights", "absorb_output_weights",
    "output_project", "streaming_kept", "mla_decode_streaming", "mla_cache_elems_per_token",
    "mha_cache_elems_per_token", "gqa_cache_elems_per_token",
    "mqa_cache_elems_per_token", "gqa_equivalent_groups",
]
