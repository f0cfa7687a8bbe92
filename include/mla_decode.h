/*
 * mla_decode.h — C ABI of the MI355X (gfx950) MLA paged-decode library.
 *
 * Multi-Head Latent Attention decode over a compressed, paged latent KV cache.
 * The method is the one described on the page "Multi-Head Latent Attention:
 * Scaling LLM Serving Throughput via Low-Rank KV Compression" (priorstack.com):
 *   - the cache keeps, per token, only the latent c^KV (d_c values) and the
 *     decoupled rotary key k^R (d_h^R values) — section "Empirical Gains",
 *     paragraph on what MLA caches, and FAQ "What does MLA store in the KV
 *     cache per token?";
 *   - at inference W^UK is absorbed into the query side and W^UV into the
 *     output side, so per-head keys and values are never materialised — same
 *     section, paragraph on absorption, and FAQ "How does MLA optimize
 *     computation during inference?";
 *   - only the decoupled rotary parts carry position (decoupled RoPE), which
 *     is what keeps the content path linear — same section.
 * The rotary embedding rotates adjacent coordinate pairs by position-scaled
 * angles ("Deepseek-V3 Define 1: Higher Attachment of Head", dataforcee.us,
 * rotary-embedding part) and runs in FP32 ("Multi-Head Latent Attention –
 * Latent KV-Cache (DeepSeek v3)", eeumee.net, "FP8/FP32 Mixed Precision").
 *
 * One decode step is three calls on the caller's stream (after mla_append_kv
 * has written the step's new tokens into the cache):
 *   mla_absorb_q      q~ = W_UK[h]^T q^C per head, and q_pe = RoPE(q^R) in fp32
 *   mla_decode_paged  split-KV attention of [q~; q_pe] over [c^KV; k^R] through
 *                     the block table; writes per-split partial results into
 *                     the caller's workspace
 *   mla_combine       merges the splits (log-sum-exp weights) into the latent
 *                     output o~ = sum_t p_t c_t, then optionally o = W_UV[h] o~
 *
 * Conventions (all entry points):
 *   - Every pointer argument is a DEVICE pointer unless its comment says
 *     "host".  The caller allocates and owns every buffer; the library never
 *     allocates, keeps no state between calls, and never synchronises the
 *     host with the device.
 *   - Tensors are dense, row-major (last dimension contiguous), and every
 *     device pointer must be 16-byte aligned.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and runs asynchronously; outputs are ready once the stream reaches them.
 *   - Every call returns an mla_status_t.  Argument checks (null pointers,
 *     alignment, shapes, dtype combinations, workspace size) run on the host
 *     before anything is enqueued; a call that returns an error has enqueued
 *     nothing.  MLA_ERR_HIP reports a failed launch.
 *   - Device-side preconditions that are NOT checked (the host cannot see
 *     device memory without a sync): 0 <= block_table entries < num_pages for
 *     every page a sequence uses; 0 <= seqlens[b] <= max_seqlen <=
 *     max_pages_per_seq * page_size.  A row whose query has no visible key
 *     (seqlens[b] - q_len + j < 0) outputs zeros and LSE = -inf.
 *
 * Supported shapes and dtypes (anything else returns MLA_ERR_UNSUPPORTED):
 *   - act BF16, latent BF16 or FP8_E4M3: d_latent = 512, d_rope = 64,
 *     d_nope = 128, d_v = 128, page_size = 64, any n_heads >= 1.
 *   - act F32, latent F32: d_latent <= 128 and a multiple of 16,
 *     d_rope <= 32 and even, d_nope <= 128, d_v <= 128, page_size = 64.
 *   - q_len in [1, 8]; batch >= 0 (batch = 0 is a no-op).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,
  MLA_ERR_BAD_SHAPE = 2,
  MLA_ERR_BAD_DTYPE = 3,
  MLA_ERR_MISALIGNED = 4,
  MLA_ERR_WORKSPACE_TOO_SMALL = 5,
  MLA_ERR_UNSUPPORTED = 6,
  MLA_ERR_HIP = 7
} mla_status_t;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2 /* OCP e4m3 ("e4m3fn"), largest finite 448, no infinities */
} mla_dtype_t;

/* Problem dimensions, passed by (host) pointer to every call. */
typedef struct {
  int32_t n_heads;      /* n_h, query heads                                  */
  int32_t d_latent;     /* d_c, width of the cached latent c^KV              */
  int32_t d_rope;       /* d_h^R, width of the decoupled rotary key/query    */
  int32_t d_nope;       /* width of the content query q^C (rows of W_UK[h])  */
  int32_t d_v;          /* width of each head's value/output (rows of W_UV[h]) */
  int32_t page_size;    /* tokens per cache page                             */
  float softmax_scale;  /* multiplies q.k before the softmax                 */
  float rope_base;      /* rotary base: theta_i = base^(-2i/d_rope)          */
  int32_t act_dtype;    /* mla_dtype_t of q, W_UK, W_UV, k^R and outputs     */
  int32_t latent_dtype; /* mla_dtype_t of the cached latent c^KV             */
} mla_dims_t;

/*
 * Absorb the content query into latent space and rotate the rotary query.
 *   q_nope   [batch, q_len, n_heads, d_nope]   act dtype
 *   q_rope   [batch, q_len, n_heads, d_rope]   act dtype, not yet rotated
 *   seqlens  [batch] int32; query j of sequence b sits at position
 *            seqlens[b] - q_len + j (its own token is already in the cache)
 *   w_uk     [n_heads, d_nope, d_latent]       act dtype; row n of W_UK[h]
 *            maps the latent to content-key coordinate n
 *   q_latent out [batch, q_len, n_heads, d_latent]:
 *            act dtype for BF16/F32 latents; for FP8_E4M3 latents, e4m3 codes
 *            of q~ / q_latent_scale
 *   q_latent_scale out [batch, q_len, n_heads] f32 (FP8_E4M3 latent only,
 *            = max|q~| / 448 per row; must be NULL otherwise)
 *   q_pe     out [batch, q_len, n_heads, d_rope] act dtype: q^R with adjacent
 *            pairs (x_2i, x_2i+1) rotated by pos * rope_base^(-2i/d_rope); the
 *            angle is formed in fp64, the rotation is done in fp32
 */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                          const void* q_nope, const void* q_rope,
                          const int32_t* seqlens, const void* w_uk,
                          void* q_latent, float* q_latent_scale, void* q_pe,
                          void* stream);

/*
 * Host-side: bytes of workspace mla_decode_paged / mla_combine need for this
 * launch shape.  `bytes` is a HOST pointer.
 */
mla_status_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch,
                                       int32_t q_len, int32_t max_seqlen,
                                       size_t* bytes);

/*
 * Split-KV attention of the absorbed query over the paged latent cache.
 * Score of cached token t for row (b, j, h):
 *     s = softmax_scale * ( q~[b,j,h] . c_t  +  q_pe[b,j,h] . k^R_t ),
 * with c_t = kv_scale[t] * code_t for FP8_E4M3 latents.  With causal != 0,
 * query j sees tokens t <= seqlens[b] - q_len + j; otherwise all seqlens[b].
 *   q_latent, q_latent_scale, q_pe   as written by mla_absorb_q
 *   kv_latent [num_pages, page_size, d_latent]  latent dtype
 *   kv_scale  [num_pages, page_size] f32 (FP8_E4M3 latent only, else NULL)
 *   kv_rope   [num_pages, page_size, d_rope]    act dtype, k^R stored already
 *             rotated at its own position
 *   block_table [batch, max_pages_per_seq] int32: token t of sequence b is in
 *             page block_table[b, t / page_size] at slot t % page_size
 *   seqlens   [batch] int32, tokens in cache per sequence
 *   max_seqlen  host-side upper bound of seqlens (sizes the launch)
 *   workspace   at least mla_decode_workspace_size() bytes; receives the
 *             per-split partial outputs and log-sum-exps read by mla_combine
 * Unused cache slots and pages may hold anything (NaN included).  Latent and
 * rotary rows past a sequence's end are never read; the FP8 scales of the
 * unused slots of a page the sequence uses are read with their tile and never
 * reach a result (their tokens' weights are set to zero first).
 */
mla_status_t mla_decode_paged(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                              int32_t causal, const void* q_latent,
                              const float* q_latent_scale, const void* q_pe,
                              const void* kv_latent, const float* kv_scale,
                              const void* kv_rope, int32_t num_pages,
                              const int32_t* block_table, int32_t max_pages_per_seq,
                              const int32_t* seqlens, int32_t max_seqlen,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Merge the splits written by mla_decode_paged (same dims, batch, q_len,
 * seqlens, max_seqlen and workspace).
 *   lse = log(sum_s exp(lse_s)),  o~ = sum_s exp(lse_s - lse) * o~_s   (natural log)
 *   w_uv  [n_heads, d_v, d_latent] act dtype, or NULL
 *   out   w_uv != NULL: [batch, q_len, n_heads, d_v] act dtype, out = W_UV[h] o~
 *         w_uv == NULL: [batch, q_len, n_heads, d_latent] act dtype, out = o~
 *   lse   [batch, q_len, n_heads] f32, or NULL
 */
mla_status_t mla_combine(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                         const void* workspace, size_t workspace_bytes,
                         const int32_t* seqlens, int32_t max_seqlen,
                         const void* w_uv, void* out, float* lse, void* stream);

/*
 * Append the new tokens of a decode step to the paged cache (run it before
 * the step's mla_decode_paged).  New token j of sequence b sits at position
 * pos = seqlens[b] - q_len + j (the lengths already count the new tokens);
 * it is written at page block_table[b, pos / page_size], slot
 * pos % page_size:
 *   - latent: c = kv_c[b, j] / sqrt(mean(kv_c[b, j]^2) + norm_eps) * norm_weight,
 *     computed in fp32 (RMSNorm of the compressed key/value in FP32: "FP8
 *     Mixed-Precision Training", eeumee.net, "Three Main Architectures"),
 *     stored in the latent dtype.  FP8_E4M3: kv_scale[row] = max|c| / 448
 *     (1 for an all-zero row) and codes = e4m3(c / kv_scale[row]), rounded to
 *     nearest-even, saturated at +-448 ("Multi-Head Latent Attention – Latent
 *     KV-Cache (DeepSeek v3)", "FP8/FP32 Mixed Precision");
 *   - rotary key: k_rope[b, j] with adjacent pairs rotated by
 *     pos * rope_base^(-2i/d_rope) (angle in fp64, rotation in fp32), stored
 *     in the act dtype: the decode reads k^R already rotated.
 * A token with pos < 0 is not written.
 *   kv_c        [batch, q_len, d_latent] act dtype, the latent before RMSNorm
 *   k_rope      [batch, q_len, d_rope]   act dtype, not rotated
 *   norm_weight [d_latent]               act dtype, the RMSNorm gain
 *   norm_eps    > 0
 *   seqlens, block_table, max_pages_per_seq, num_pages   as for mla_decode_paged
 *   kv_latent, kv_scale (FP8_E4M3 latent only, else NULL), kv_rope: the cache,
 *               modified in place at the new tokens' slots only
 * Ownership and errors as for every call.  The same device preconditions
 * apply; a table entry outside [0, num_pages) or a position past
 * max_pages_per_seq * page_size is a broken precondition, for which the
 * kernel writes nothing for that token.
 */
mla_status_t mla_append_kv(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                           const void* kv_c, const void* k_rope, const void* norm_weight,
                           float norm_eps, const int32_t* seqlens,
                           const int32_t* block_table, int32_t max_pages_per_seq,
                           void* kv_latent, float* kv_scale, void* kv_rope,
                           int32_t num_pages, void* stream);

/* Static, human-readable name of a status code. */
const char* mla_status_string(mla_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
