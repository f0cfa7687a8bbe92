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
 *   - Device-side preconditions, not checked by default (the host cannot see
 *     device memory without a sync): 0 <= block_table entries < num_pages for
 *     every page a sequence uses; 0 <= seqlens[b] <= max_seqlen <=
 *     max_pages_per_seq * page_size; for FP8_E4M3 latents, the scale of every
 *     visible token is a normal positive number (an all-zero latent row
 *     carries any such scale: mla_append_kv writes 1; a zero scale is not
 *     accepted).  A row whose query has no visible key
 *     (seqlens[b] - q_len + j < 0) outputs zeros and LSE = -inf.
 *   - Validation mode: with the environment variable MLA_VALIDATE set to "1"
 *     (read on every call), mla_decode_paged first checks the lengths and
 *     block-table preconditions on the device, waits for that check (the one
 *     host synchronisation in the library) and returns MLA_ERR_BAD_SHAPE,
 *     having launched no decode, if any sequence breaks one.
 *     mla_validate_paged_host runs the same check on host copies.
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
  MLA_ERR_HIP = 7,
  MLA_ERR_SCRATCH_TOO_SMALL = 8
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
 *            one power of two per row: the smallest 2^k with
 *            max|q~| / 2^k <= 448, 1 for an all-zero row; must be NULL
 *            otherwise)
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
 * StreamingLLM-style eviction view of the paged cache (the related-papers
 * page "Related papers: SnapMLA: Efficient Long-Context MLA Decoding via H…",
 * scifaro.com, names such eviction techniques, StreamingLLM and SnapKV, for
 * bounding a long context's KV cache).  A sequence of L tokens keeps its first
 * sink_pages pages and its most recent tokens from the page boundary at or
 * below L - window_pages * page_size on; a sequence whose window would reach
 * back into its sinks keeps everything.  Kept tokens are not moved and keep
 * the positions they were cached at; the view is a new block table and new
 * lengths, written on the device:
 *   out_seqlens[b]      = tokens kept (sink_pages * page_size + L - start, or L)
 *   out_block_table[b]  = the kept pages in order (sink pages, then window
 *                         pages), 0 in the unused columns
 * A decode step over the view runs mla_absorb_q with the TRUE seqlens (the
 * query positions), then mla_decode_paged and mla_combine with out_seqlens,
 * out_block_table, max_pages_out and a max_seqlen of at most
 * max_pages_out * page_size; every kept token's score is its score in the full
 * cache, so the result is attention restricted to the kept keys.
 *   seqlens, block_table [batch, max_pages_per_seq]   as for mla_decode_paged
 *   sink_pages >= 0, window_pages >= 1
 *   out_seqlens [batch] int32, out_block_table [batch, max_pages_out] int32:
 *     device, written; max_pages_out >= sink_pages + window_pages + 1
 * Errors: MLA_ERR_BAD_SHAPE for counts out of range, MLA_ERR_NULL_POINTER,
 * MLA_ERR_HIP for a failed launch.  The same device preconditions as the
 * decode apply to seqlens and block_table.
 */
mla_status_t mla_streaming_view(const mla_dims_t* dims, int32_t batch,
                                const int32_t* seqlens, const int32_t* block_table,
                                int32_t max_pages_per_seq, int32_t sink_pages,
                                int32_t window_pages, int32_t* out_seqlens,
                                int32_t* out_block_table, int32_t max_pages_out,
                                void* stream);

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

/*
 * Host-side check of the paged decode's device preconditions on HOST copies
 * of the lengths and the block table (the check MLA_VALIDATE=1 runs on the
 * device before a decode).  Sequence b passes when 0 <= seqlens[b] <=
 * max_seqlen, seqlens[b] <= max_pages_per_seq * page_size, and
 * 0 <= block_table[b, k] < num_pages for every page k < ceil(seqlens[b] /
 * page_size) (entries past those pages are never read and may hold anything).
 *   block_table  HOST [batch, max_pages_per_seq] int32
 *   seqlens      HOST [batch] int32
 *   bad          HOST out: the number of sequences that fail
 * Returns MLA_OK when every sequence passes, MLA_ERR_BAD_SHAPE when some
 * fail (or an argument is out of range), MLA_ERR_NULL_POINTER for a NULL
 * pointer.  Touches no device.
 */
mla_status_t mla_validate_paged_host(const mla_dims_t* dims, int32_t batch, int32_t num_pages,
                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                     const int32_t* seqlens, int32_t max_seqlen, int32_t* bad);

/*
 * Allocation-free decode: mla_decode_paged followed by mla_combine, with the
 * split partials kept in a static device array of the library instead of a
 * caller workspace.  For callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It calls no hipMalloc, hipFree or other allocating routine;
 * the caller still passes (and owns) every input and output.
 *   Arguments: as for mla_decode_paged and mla_combine (same meaning, layout
 *   and preconditions; out/lse as for mla_combine, w_uv may be NULL for the
 *   latent output).
 *   Scratch: MLA_NOALLOC_SCRATCH_BYTES (80 MiB) per device, held by each GPU
 *   the library runs on until the process ends.  A launch shape needs
 *   mla_decode_workspace_size() bytes of it (at 256 compute units, up to
 *   about 600 partial slots of 128 rows: B * ceil(q_len * n_heads / 128) +
 *   256 <= ~600, e.g. 128 sequences x 2 query tokens x 128 heads); a larger
 *   one returns MLA_ERR_SCRATCH_TOO_SMALL having enqueued nothing.
 *   Concurrency: every call on one GPU uses that GPU's single scratch, so
 *   calls that overlap on one GPU (other streams, other host threads) race
 *   and must be serialised by the caller.  Nothing in the scratch needs
 *   clearing between calls: each decode writes everything its merge reads.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (80u * 1024u * 1024u)
mla_status_t mla_decode_noalloc(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                int32_t causal, const void* q_latent,
                                const float* q_latent_scale, const void* q_pe,
                                const void* kv_latent, const float* kv_scale,
                                const void* kv_rope, int32_t num_pages,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* seqlens, int32_t max_seqlen, const void* w_uv,
                                void* out, float* lse, void* stream);

/*
 * Many query tokens per sequence (chunked prefill, verification of several
 * drafted tokens) in the NON-absorbed form: the other of the two
 * functionally equivalent MLA kernel formulations ("Related papers: SnapMLA:
 * Efficient Long-Context MLA Decoding via H…", scifaro.com, the abstract on
 * two formulations).  Per head, the content keys and values are expanded
 * from the cached latent, K^C_t = W_UK[h] c_t and V_t = W_UV[h] c_t ("Multi-
 * Head Latent Attention: Scaling LLM Serving Throughput via Low-Rank KV
 * Compression", "Empirical Gains"), then ordinary causal attention runs:
 *     s = softmax_scale * ( q^C . K^C_t + R(pos_j) q^R . k^R_t ),
 *     out[b, j, h] = sum_{t <= pos_j} softmax(s)_t V_t,
 * with pos_j = seqlens[b] - q_len + j (the chunk's tokens are already in the
 * cache).  The result equals mla_absorb_q + mla_decode_paged(causal) +
 * mla_combine(w_uv) up to rounding; with many query rows it does less
 * arithmetic (2 d_c (d_nope + d_v) per key and head once, then
 * 2 (d_nope + d_R + d_v) per key and row).
 *   q_nope [batch, q_len, n_heads, d_nope] act; q_rope [batch, q_len,
 *          n_heads, d_rope] act, not rotated (rotated here in fp32)
 *   kv_latent, kv_rope, num_pages, block_table, max_pages_per_seq, seqlens,
 *          max_seqlen: the paged cache, as for mla_decode_paged
 *   w_uk, w_uv [n_heads, 128, d_latent] act
 *   workspace  >= mla_prefill_workspace_size() bytes: the expanded K^C and V
 *          [batch, n_heads, ceil(max_seqlen / 64) * 64, 128] bf16 each
 *   out   [batch, q_len, n_heads, d_v] act;  lse [batch, q_len, n_heads] f32
 *          natural log, or NULL.  A row with no visible key outputs zeros and
 *          LSE = -inf.
 * Supported: act BF16 and latent BF16 at the decode path's dims;
 * 1 <= q_len <= 65536.  Errors, preconditions and MLA_VALIDATE as for
 * mla_decode_paged.
 */
mla_status_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t batch,
                                        int32_t max_seqlen, size_t* bytes);
mla_status_t mla_prefill_paged(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                               const void* q_nope, const void* q_rope, const void* kv_latent,
                               const void* kv_rope, int32_t num_pages,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               const int32_t* seqlens, int32_t max_seqlen, const void* w_uk,
                               const void* w_uv, void* workspace, size_t workspace_bytes,
                               void* out, float* lse, void* stream);

/*
 * Dense products around the attention: the latent down-projections of the
 * hidden state ("Multi-Head Latent Attention – Latent KV-Cache (DeepSeek
 * v3)", eeumee.net, "Operation Flow", step 1: c^Q, c^KV from h), the query
 * up-projection (step 2) and the weight-level absorption of W^UK into the
 * query weights and of W^UV into the output projection W^O ("Multi-Head
 * Latent Attention: Scaling LLM Serving Throughput via Low-Rank KV
 * Compression", "Empirical Gains", the paragraph on absorption).
 *
 * mla_gemm_bf16: C[b] = A[b] B[b]^T for b < batch, bf16 inputs, fp32
 *   accumulation.  A [m, lda] and B [n, ldb] are row-major with the k
 *   dimension contiguous (lda, ldb >= k, multiples of 8; k a multiple of 8);
 *   C [m, ldc] row-major in c_dtype (MLA_BF16, rounded to nearest even, or
 *   MLA_F32); stride_* in elements between batch entries (0 shares an
 *   operand).  A and B 16-byte aligned, C 4-byte aligned.  A down-projection
 *   c = W^D h of T tokens is mla_gemm_bf16(1, T, d_out, d_model, h, d_model,
 *   0, W^D, d_model, 0, c, ...).
 */
mla_status_t mla_gemm_bf16(int32_t batch, int32_t m, int32_t n, int32_t k, const void* a,
                           int64_t lda, int64_t stride_a, const void* b, int64_t ldb,
                           int64_t stride_b, void* c, int32_t c_dtype, int64_t ldc,
                           int64_t stride_c, void* stream);

/*
 * Weight-level absorption (bf16 activations), done once per set of weights:
 *   mla_absorb_query_weights:  W~[h] = W_UK[h]^T W_UQ[h]
 *       w_uq [n_heads, d_nope, d_cq], w_uk [n_heads, d_nope, d_latent]
 *       -> w_q_absorbed [n_heads, d_latent, d_cq] (bf16), so that the absorbed
 *       query of a token is q~[h] = W~[h] c^Q (mla_query_from_latent);
 *   mla_absorb_output_weights: W~O[:, h d_latent + c] = sum_v W_O[:, h d_v + v] W_UV[h][v][c]
 *       w_o [d_model, n_heads d_v], w_uv [n_heads, d_v, d_latent]
 *       -> w_o_absorbed [d_model, n_heads d_latent] (bf16), so that the layer
 *       output is y = W~O [o~_1; ...; o~_H] from the latent outputs o~ that
 *       mla_combine writes with w_uv = NULL (one mla_gemm_bf16).
 * workspace: >= mla_absorb_weights_workspace_size() bytes (transposed weight
 * copies).  d_cq a multiple of 8.
 */
mla_status_t mla_absorb_weights_workspace_size(const mla_dims_t* dims, int32_t d_cq,
                                               size_t* bytes);
mla_status_t mla_absorb_query_weights(const mla_dims_t* dims, int32_t d_cq, const void* w_uq,
                                      const void* w_uk, void* w_q_absorbed, void* workspace,
                                      size_t workspace_bytes, void* stream);
mla_status_t mla_absorb_output_weights(const mla_dims_t* dims, int32_t d_model, const void* w_o,
                                       const void* w_uv, void* w_o_absorbed, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * The decode query from the query latent through absorbed weights (in place
 * of mla_absorb_q when W_UK has been folded into the query weights):
 *   q_latent[b, j, h] = W~[h] c_q[b, j]          (W~ from mla_absorb_query_weights)
 *   q_pe[b, j, h]     = R(pos_j) (W_QR c_q[b, j])[h d_rope ..]   (fp32 rotation,
 *                       pos_j = seqlens[b] - q_len + j, as mla_absorb_q)
 *   c_q [batch, q_len, d_cq] bf16; w_q_absorbed [n_heads, d_latent, d_cq];
 *   w_qr [n_heads d_rope, d_cq]; q_latent [batch, q_len, n_heads, d_latent];
 *   q_pe [batch, q_len, n_heads, d_rope].  BF16 latents only.
 */
mla_status_t mla_query_from_latent(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                   int32_t d_cq, const void* c_q, const void* w_q_absorbed,
                                   const void* w_qr, const int32_t* seqlens, void* q_latent,
                                   void* q_pe, void* stream);

/* Static, human-readable name of a status code. */
const char* mla_status_string(mla_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
