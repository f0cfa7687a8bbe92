// Split combine and output up-projection, gfx950.
//
// For each (sequence b, query j, head h) the decode pass left one partial per
// chunk of its cache: o~_s (normalised) and lse_s (natural log).  Merging them
// is the log-sum-exp identity
//     lse = log sum_s exp(lse_s),   o~ = sum_s exp(lse_s - lse) o~_s,
// which reproduces softmax over the whole cache exactly.  The up-projection
// o = W_UV[h] o~ is the value side of weight absorption ("Multi-Head Latent
// Attention: Scaling LLM Serving Throughput via Low-Rank KV Compression",
// section "Empirical Gains", paragraph on absorbing W^UV into the output
// projection): values are never expanded per token, only the one merged
// latent per head is.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

// First chunk (= partial slot) of unit (b, rg) and its chunk count, as the
// decode pass recorded them (a sequence with no cached token has no chunk).
__device__ __forceinline__ void unit_slots(const CombineArgs& a, int b, int rg, int& first,
                                           int& count) {
  if (a.seqlens[b] <= 0) {
    first = 0;
    count = 0;
    return;
  }
  const int64_t u = (int64_t)b * a.row_groups + rg;
  first = a.unit_chunks[2 * u];
  count = a.unit_chunks[2 * u + 1];
}

// Merge one 64-dim slice [64 sl, 64 sl + 64) of one row's partials (one
// thread).  Partials are bf16 when the activations are bf16 and f32
// otherwise.  Returns the row's log-sum-exp (-inf: no visible key, acc = 0).
constexpr int SLICE = 64;

__device__ __forceinline__ void load_slice(const CombineArgs& a, int64_t slot, int r, int sl,
                                           float (&v)[SLICE]) {
  if (a.out_dtype == DT_BF16) {
    const uint16_t* src = (const uint16_t*)a.part_o + (slot * kRowsPerWG + r) * a.d_lat + sl * SLICE;
#pragma unroll
    for (int c = 0; c < SLICE / 8; ++c) {
      const u32x4 u = *(const u32x4*)(src + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[c * 8 + 2 * e] = __uint_as_float(u[e] << 16);
        v[c * 8 + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
  } else {
    const float* src = (const float*)a.part_o + (slot * kRowsPerWG + r) * a.d_lat + sl * SLICE;
#pragma unroll
    for (int c = 0; c < SLICE / 4; ++c) {
      const f32x4 u = *(const f32x4*)(src + c * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[c * 4 + e] = u[e];
    }
  }
}

__device__ __forceinline__ float merge_slice(const CombineArgs& a, int first, int count, int r,
                                             int sl, float (&acc)[SLICE]) {
#pragma unroll
  for (int e = 0; e < SLICE; ++e) acc[e] = 0.f;
  float mx = -INFINITY;
  for (int s = 0; s < count; ++s)
    mx = fmaxf(mx, a.part_lse[(int64_t)(first + s) * kRowsPerWG + r]);
  if (mx == -INFINITY) return -INFINITY;
  float tot = 0.f;
  for (int s = 0; s < count; ++s) {
    const float ls = a.part_lse[(int64_t)(first + s) * kRowsPerWG + r];
    if (ls == -INFINITY) continue;
    const float wgt = __expf(ls - mx);
    tot += wgt;
    float v[SLICE];
    load_slice(a, first + s, r, sl, v);
#pragma unroll
    for (int e = 0; e < SLICE; ++e) acc[e] += wgt * v[e];
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int e = 0; e < SLICE; ++e) acc[e] *= inv;
  return mx + __logf(tot);
}

// out = o~ (latent output): a workgroup merges 32 rows, thread = (row, slice).
constexpr int ROWS_PER_WG = 32;

__global__ __launch_bounds__(256) void combine_latent_kernel(CombineArgs a) {
  const int ml = threadIdx.x / 8, sl = threadIdx.x % 8;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_WG + ml;
  const int64_t rows = (int64_t)a.batch * a.q_len * a.n_heads;
  if (row >= rows || sl * SLICE >= a.d_lat) return;
  const int b = (int)(row / ((int64_t)a.q_len * a.n_heads));
  const int jh = (int)(row % ((int64_t)a.q_len * a.n_heads));
  int first, count;
  unit_slots(a, b, jh / kRowsPerWG, first, count);
  float acc[SLICE];
  const float lse = merge_slice(a, first, count, jh % kRowsPerWG, sl, acc);
  if (a.out_dtype == DT_BF16) {
    uint16_t* o = (uint16_t*)a.out + row * a.d_lat + sl * SLICE;
#pragma unroll
    for (int c = 0; c < SLICE / 8; ++c)
      *(u32x4*)(o + c * 8) = u32x4{pack_bf16x2(acc[c * 8], acc[c * 8 + 1]),
                                   pack_bf16x2(acc[c * 8 + 2], acc[c * 8 + 3]),
                                   pack_bf16x2(acc[c * 8 + 4], acc[c * 8 + 5]),
                                   pack_bf16x2(acc[c * 8 + 6], acc[c * 8 + 7])};
  } else {
    float* o = (float*)a.out + row * a.d_lat + sl * SLICE;
#pragma unroll
    for (int c = 0; c < SLICE / 4; ++c)
      *(f32x4*)(o + c * 4) = f32x4{acc[c * 4], acc[c * 4 + 1], acc[c * 4 + 2], acc[c * 4 + 3]};
  }
  if (a.lse != nullptr && sl == 0) a.lse[row] = lse;
}

// bf16: out[m, h, :] = W_UV[h] o~[m, h, :] for a block of 32 rows m = (b, j)
// of one head.  Merged rows go to LDS as bf16; the product runs on
// v_mfma_f32_16x16x32_bf16 as D^T = W_UV[h] o~^T, A = W rows (global, 16-byte
// loads), B = o~ rows (LDS).
constexpr int UV_M = 32;
constexpr int UV_DLAT = 512;
constexpr int UV_DV = 128;

__global__ __launch_bounds__(256) void combine_uv_bf16_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_o[UV_M][UV_DLAT + 8];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
  // blocks of one head are adjacent in the logical order (shared W_UV in L2)
  const int blk = xcd_logical_id(blockIdx.x, gridDim.x);
  const int h = blk / nmb;
  const int mb = blk % nmb;
  const int m_total = a.batch * a.q_len;

  // 1. merge the block's rows into LDS: thread = (row, 64-dim slice)
  {
    const int ml = threadIdx.x / 8, sl = threadIdx.x % 8;
    const int m = mb * UV_M + ml;
    float acc[SLICE];
    float lse = -INFINITY;
    if (m < m_total) {
      const int b = m / a.q_len, j = m % a.q_len;
      const int jh = j * a.n_heads + h;
      int first, count;
      unit_slots(a, b, jh / kRowsPerWG, first, count);
      lse = merge_slice(a, first, count, jh % kRowsPerWG, sl, acc);
    } else {
#pragma unroll
      for (int e = 0; e < SLICE; ++e) acc[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < SLICE / 8; ++c)
      *(u32x4*)&s_o[ml][sl * SLICE + c * 8] =
          u32x4{pack_bf16x2(acc[c * 8], acc[c * 8 + 1]), pack_bf16x2(acc[c * 8 + 2], acc[c * 8 + 3]),
                pack_bf16x2(acc[c * 8 + 4], acc[c * 8 + 5]), pack_bf16x2(acc[c * 8 + 6], acc[c * 8 + 7])};
    if (a.lse != nullptr && sl == 0 && m < m_total) a.lse[(int64_t)m * a.n_heads + h] = lse;
  }
  __syncthreads();

  // 2. D^T[n, m] = sum_k W[h, n, k] o~[m, k]; wave w: n blocks 2w, 2w+1; m blocks 0, 1
  const uint16_t* W = (const uint16_t*)a.w_uv + (int64_t)h * UV_DV * UV_DLAT;
  f32x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int kk = 0; kk < UV_DLAT / 32; ++kk) {
    u16x8 wa[2], ob[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
      wa[x] = *(const u16x8*)(W + (int64_t)((2 * w + x) * 16 + lr) * UV_DLAT + kk * 32 + lg * 8);
#pragma unroll
    for (int y = 0; y < 2; ++y) ob[y] = *(const u16x8*)&s_o[y * 16 + lr][kk * 32 + lg * 8];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = mfma_bf16_16x16x32(wa[x], ob[y], acc[x][y]);
  }
  // lane holds D^T[n = nblk*16 + lg*4 + r][m = mblk*16 + lr]
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int m = mb * UV_M + y * 16 + lr;
    if (m >= m_total) continue;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int n0 = (2 * w + x) * 16 + lg * 4;
      uint16_t* o = (uint16_t*)a.out + ((int64_t)m * a.n_heads + h) * UV_DV + n0;
      *(u32x2*)o = u32x2{pack_bf16x2(acc[x][y][0], acc[x][y][1]),
                         pack_bf16x2(acc[x][y][2], acc[x][y][3])};
    }
  }
}

// f32 (small shapes: d_lat <= 512, d_v <= 128): one workgroup per (head, 32 rows),
// merged rows in LDS, plain fp32 FMAs.
__global__ __launch_bounds__(256) void combine_uv_f32_kernel(CombineArgs a) {
  __shared__ float s_o[UV_M][UV_DLAT + 4];
  const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
  const int h = blockIdx.x / nmb;
  const int mb = blockIdx.x % nmb;
  const int m_total = a.batch * a.q_len;
  {
    const int ml = threadIdx.x / 8, sl = threadIdx.x % 8;
    const int m = mb * UV_M + ml;
    if (sl * SLICE < a.d_lat) {
      float acc[SLICE];
      float lse = -INFINITY;
      if (m < m_total) {
        const int b = m / a.q_len, j = m % a.q_len;
        const int jh = j * a.n_heads + h;
        int first, count;
        unit_slots(a, b, jh / kRowsPerWG, first, count);
        lse = merge_slice(a, first, count, jh % kRowsPerWG, sl, acc);
      } else {
#pragma unroll
        for (int e = 0; e < SLICE; ++e) acc[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < SLICE; ++e) s_o[ml][sl * SLICE + e] = acc[e];
      if (a.lse != nullptr && sl == 0 && m < m_total) a.lse[(int64_t)m * a.n_heads + h] = lse;
    }
  }
  __syncthreads();
  const float* W = (const float*)a.w_uv + (int64_t)h * a.d_v * a.d_lat;
  for (int idx = threadIdx.x; idx < UV_M * a.d_v; idx += blockDim.x) {
    const int ml = idx / a.d_v, n = idx % a.d_v;
    const int m = mb * UV_M + ml;
    if (m >= m_total) continue;
    float s = 0.f;
    for (int k = 0; k < a.d_lat; ++k) s = fmaf(W[(int64_t)n * a.d_lat + k], s_o[ml][k], s);
    ((float*)a.out)[((int64_t)m * a.n_heads + h) * a.d_v + n] = s;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.q_len * a.n_heads;
  if (rows == 0) return hipSuccess;
  if (a.w_uv == nullptr) {
    hipLaunchKernelGGL(combine_latent_kernel, dim3((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)),
                       dim3(256), 0, s, a);
  } else {
    const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
    const unsigned grid = (unsigned)(nmb * a.n_heads);
    if (a.out_dtype == DT_BF16)
      hipLaunchKernelGGL(combine_uv_bf16_kernel, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(combine_uv_f32_kernel, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
