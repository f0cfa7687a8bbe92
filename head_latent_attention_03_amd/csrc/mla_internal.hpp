// Launch arguments passed from the C ABI layer to the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

struct AbsorbArgs {
  const void* q_nope;
  const void* q_rope;
  const int32_t* seqlens;
  const void* w_uk;
  void* q_lat;
  float* q_lat_scale;
  void* q_pe;
  int32_t batch, q_len, n_heads, d_nope, d_lat, d_rope;
  float rope_base;
};

struct DecodeArgs {
  const void* q_lat;
  const float* q_scale;      // fp8 latent only
  const void* q_pe;
  const void* kv_lat;
  const float* kv_scale;     // fp8 latent only
  const void* kv_rope;
  const int32_t* block_table;
  const int32_t* seqlens;
  void* part_o;              // [slots, 128, d_lat] bf16 (bf16 activations) or f32
  float* part_lse;           // [slots, 128]        f32 (natural log)
  int32_t* unit_chunks;      // [units, 2]: first chunk and chunk count of each unit
  int32_t max_pages, batch, q_len, n_heads, causal;
  int32_t d_lat, d_rope;
  int32_t num_wg, row_groups;
  float scale_log2;          // softmax_scale * log2(e)
};

struct CombineArgs {
  const void* part_o;        // bf16 when out_dtype is bf16, else f32
  const float* part_lse;
  const int32_t* unit_chunks;  // [units, 2] as written by the decode pass
  const int32_t* seqlens;
  const void* w_uv;          // may be null
  void* out;
  float* lse;                // may be null
  int32_t batch, q_len, n_heads, d_lat, d_v;
  int32_t num_wg, row_groups;
  int32_t out_dtype;         // Dt
};

hipError_t launch_absorb_bf16(const AbsorbArgs& a, bool fp8_out, hipStream_t s);
hipError_t launch_absorb_f32(const AbsorbArgs& a, hipStream_t s);
// grid = launched workgroups (an upper bound of the plan's chunk count)
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, int grid);
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s, int grid);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s, int grid);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);


struct AppendArgs {
  const void* kv_c;          // [batch, q_len, d_lat] act dtype, before RMSNorm
  const void* k_rope;        // [batch, q_len, d_rope] act dtype, not rotated
  const void* norm_weight;   // [d_lat] act dtype
  const int32_t* seqlens;
  const int32_t* block_table;
  void* kv_lat;              // [num_pages, page_size, d_lat] latent dtype
  float* kv_scale;           // [num_pages, page_size] (e4m3 latent only)
  void* kv_rope;             // [num_pages, page_size, d_rope] act dtype
  int32_t batch, q_len, d_lat, d_rope, page_size, max_pages, num_pages;
  int32_t act_dtype, lat_dtype;  // Dt
  float eps, rope_base;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);

struct ValidateArgs {
  const int32_t* block_table;  // [batch, max_pages]
  const int32_t* seqlens;      // [batch]
  int32_t* bad;                // out: sequences that break a precondition
  int32_t batch, max_pages, max_seqlen, page_size, num_pages;
};

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s);

struct StreamingViewArgs {
  const int32_t* seqlens;
  const int32_t* block_table;
  int32_t* out_seqlens;
  int32_t* out_block_table;
  int32_t batch, max_pages, max_pages_out, page_size, sink_pages, window_pages;
};

hipError_t launch_streaming_view(const StreamingViewArgs& a, hipStream_t s);

struct GemmArgs {            // C[b] = A[b] B[b]^T, bf16 in, fp32 accumulate
  const void* a;             // [batch][m][lda] bf16 (k contiguous)
  const void* b;             // [batch][n][ldb] bf16 (k contiguous)
  void* c;                   // [batch][m][ldc] bf16 or f32
  int64_t lda, ldb, ldc, stride_a, stride_b, stride_c;   // elements
  int32_t batch, m, n, k, c_f32;
};
hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t s);
// which tile launch_gemm_nt takes (true: 256 x 160, false: 128 x 128)
bool gemm_nt_takes_wide_tiles(const GemmArgs& g);

struct TransposeArgs {       // dst[b][c][r] = src[b][r][c], 16-bit elements
  const void* src;
  void* dst;
  int32_t batch, rows, cols;
};
hipError_t launch_transpose(const TransposeArgs& t, hipStream_t s);

struct RopeArgs {            // q_pe = RoPE(q_rope) at pos = seqlens[b] - q_len + j
  const void* src;           // [batch, q_len, H, d_rope] bf16
  void* dst;                 // same shape (may equal src)
  const int32_t* seqlens;
  int32_t batch, q_len, n_heads, d_rope;
  float rope_base;
};
hipError_t launch_rope_query(const RopeArgs& r, hipStream_t s);

struct PrefillArgs {
  const void* q_nope;        // [batch, q_len, H, 128] bf16
  const void* q_rope;        // [batch, q_len, H, 64] bf16, not rotated
  const void* kv_lat;        // [num_pages, 64, 512] bf16
  const void* kv_rope;       // [num_pages, 64, 64] bf16
  const int32_t* block_table;
  const int32_t* seqlens;
  const void* w_uk;          // [H, 128, 512] bf16
  const void* w_uv;          // [H, 128, 512] bf16
  void* kexp;                // workspace [batch, H, lpad, 128] bf16: K^C
  void* vexp;                // workspace [batch, H, lpad, 128] bf16: V
  void* out;                 // [batch, q_len, H, 128] bf16
  float* lse;                // [batch, q_len, H] or null
  int32_t batch, q_len, n_heads, max_pages, lpad;
  float scale_log2, rope_base;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

}  // namespace mla
