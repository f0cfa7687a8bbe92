// Append the new tokens of a decode step to the paged latent cache, gfx950.
//
// For new token j of sequence b, at position pos = seqlens[b] - q_len + j:
//   c_t  = RMSNorm(c^KV) = c^KV / sqrt(mean(c^KV^2) + eps) * g, in fp32
//          ("FP8 Mixed-Precision Training", eeumee.net, section "Three Main
//          Architectures": the compressed key/value of MLA is normalised by
//          RMSNorm in FP32), stored in the cache's latent dtype: bf16, f32,
//          or e4m3 codes of c_t / s with s = max|c_t| / 448 per token (FP8 for
//          the products that consume it: "Multi-Head Latent Attention –
//          Latent KV-Cache (DeepSeek v3)", "FP8/FP32 Mixed Precision");
//   k^R_t = RoPE(k^R, pos), fp64 angle then fp32 rotation (same section), so
//          the decode reads the rotary key already rotated;
// written at page block_table[b, pos / page_size], slot pos % page_size.  The
// cache holds only these two per token ("Multi-Head Latent Attention:
// Scaling LLM Serving Throughput via Low-Rank KV Compression", "Empirical
// Gains", the paragraph on what MLA caches).
//
// One wave per new token; lane l handles latent coordinates l, l + 64, ...
// (coalesced row reads and writes) and rotary pair l.  The sum of squares and,
// for e4m3, the row's largest magnitude are wave reductions.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int kMaxLat = 512;              // latent coordinates per row (bf16/e4m3 path)
constexpr int kPerLane = kMaxLat / 64;
constexpr int kTokensPerWG = 4;

template <int ACT>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
  if (ACT == DT_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

template <int ACT>
__device__ __forceinline__ void store_act(void* p, int64_t i, float v) {
  if (ACT == DT_BF16) {
    ((uint16_t*)p)[i] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
  } else {
    ((float*)p)[i] = v;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = wave_sum_xor(v, m);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = wave_max_xor(v, m);
  return v;
}

template <int ACT, int LAT>
__global__ __launch_bounds__(64 * kTokensPerWG) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * kTokensPerWG + (threadIdx.x >> 6);
  if (m >= (int64_t)a.batch * a.q_len) return;
  const int b = (int)(m / a.q_len), j = (int)(m % a.q_len);
  const int pos = a.seqlens[b] - a.q_len + j;
  if (pos < 0) return;                       // the sequence holds fewer tokens than q_len
  const int pi = pos / a.page_size;
  // (out-of-range table entries are a broken precondition: nothing is written)
  if (pi >= a.max_pages) return;
  const int page = a.block_table[(int64_t)b * a.max_pages + pi];
  if (page < 0 || page >= a.num_pages) return;
  const int64_t row = (int64_t)page * a.page_size + pos % a.page_size;

  // ---- latent: RMSNorm in fp32
  float x[kPerLane];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kPerLane; ++k) {
    const int i = lane + 64 * k;
    x[k] = i < a.d_lat ? load_act<ACT>(a.kv_c, m * a.d_lat + i) : 0.f;
    ss = fmaf(x[k], x[k], ss);
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)a.d_lat + a.eps);
  float y[kPerLane];
#pragma unroll
  for (int k = 0; k < kPerLane; ++k) {
    const int i = lane + 64 * k;
    y[k] = i < a.d_lat ? x[k] * inv * load_act<ACT>(a.norm_weight, i) : 0.f;
  }
  if (LAT == DT_E4M3) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) amax = fmaxf(amax, fabsf(y[k]));
    amax = wave_max(amax);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* dst = (uint8_t*)a.kv_lat + row * a.d_lat;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int i = lane + 64 * k;
      const float v = fminf(fmaxf(y[k] / s, -448.0f), 448.0f);
      const int c = __builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false);
      if (i < a.d_lat) dst[i] = (uint8_t)(c & 0xff);
    }
    if (lane == 0) a.kv_scale[row] = s;
  } else {
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int i = lane + 64 * k;
      if (i < a.d_lat) store_act<LAT>(a.kv_lat, row * a.d_lat + i, y[k]);
    }
  }

  // ---- rotary key: pair `lane` rotated by pos * theta_lane
  if (2 * lane < a.d_rope) {
    const int64_t src = m * a.d_rope + 2 * lane;
    float y0, y1;
    rope_pair(load_act<ACT>(a.k_rope, src), load_act<ACT>(a.k_rope, src + 1), pos,
              rope_theta(lane, a.d_rope, a.rope_base), y0, y1);
    const int64_t dst = row * a.d_rope + 2 * lane;
    store_act<ACT>(a.kv_rope, dst, y0);
    store_act<ACT>(a.kv_rope, dst + 1, y1);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t tokens = (int64_t)a.batch * a.q_len;
  if (tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)((tokens + kTokensPerWG - 1) / kTokensPerWG));
  const dim3 block(64 * kTokensPerWG);
  if (a.act_dtype == DT_F32) {
    hipLaunchKernelGGL((append_kernel<DT_F32, DT_F32>), grid, block, 0, s, a);
  } else if (a.lat_dtype == DT_E4M3) {
    hipLaunchKernelGGL((append_kernel<DT_BF16, DT_E4M3>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((append_kernel<DT_BF16, DT_BF16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
