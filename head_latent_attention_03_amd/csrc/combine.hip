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

// First chunk (= partial slot) of unit (b, rg) and its chunk count.
__device__ __forceinline__ void unit_slots(const CombineArgs& a, int64_t nt, int b, int rg,
                                           int lane, int& first, int& count) {
  const int before = plan_chunks_before(a.seqlens, b, a.row_groups, nt, a.num_wg, lane);
  const int len = uni(a.seqlens[b]);
  count = plan_splits(tiles_of(len), nt, a.num_wg);
  first = before + rg * count;
}

// Merge the partials of one row into `dst` (d_lat floats or bf16), one wave.
// Lane l handles latent dims [8l, 8l + 8) (d_lat <= 512, multiple of 8).
// Returns the row's log-sum-exp.
__device__ __forceinline__ float merge_row(const CombineArgs& a, int first, int count, int r,
                                           int lane, float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float mx = -INFINITY;
  for (int s = 0; s < count; ++s) mx = fmaxf(mx, a.part_lse[(int64_t)(first + s) * kRowsPerWG + r]);
  if (mx == -INFINITY) return -INFINITY;
  float tot = 0.f;
  for (int s = 0; s < count; ++s) {
    const int64_t slot = first + s;
    const float ls = a.part_lse[slot * kRowsPerWG + r];
    if (ls == -INFINITY) continue;
    const float wgt = __expf(ls - mx);
    tot += wgt;
    if (lane * 8 < a.d_lat) {
      const float* src = a.part_o + (slot * kRowsPerWG + r) * a.d_lat + lane * 8;
      const f32x4 v0 = *(const f32x4*)src;
      const f32x4 v1 = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * v0[e];
        acc[4 + e] += wgt * v1[e];
      }
    }
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  return mx + __logf(tot);
}

// out = o~ (latent output): one wave per (b, j, h) row.
__global__ __launch_bounds__(256) void combine_latent_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.batch * a.q_len * a.n_heads;
  if (row >= rows) return;
  const int b = (int)(row / ((int64_t)a.q_len * a.n_heads));
  const int jh = (int)(row % ((int64_t)a.q_len * a.n_heads));
  const int rg = jh / kRowsPerWG, r = jh % kRowsPerWG;
  const int64_t nt = plan_total_tiles(a.seqlens, a.batch, a.row_groups, lane);
  float acc[8];
  float lse = -INFINITY;
  if (nt > 0) {
    int first, count;
    unit_slots(a, nt, b, rg, lane, first, count);
    lse = merge_row(a, first, count, r, lane, acc);
  }
  if (lse == -INFINITY) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  }
  if (lane * 8 < a.d_lat) {
    if (a.out_dtype == DT_BF16) {
      uint16_t* o = (uint16_t*)a.out + row * a.d_lat + lane * 8;
      *(u32x4*)o = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    } else {
      float* o = (float*)a.out + row * a.d_lat + lane * 8;
      *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = lse;
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
  const int64_t nt = plan_total_tiles(a.seqlens, a.batch, a.row_groups, lane);

  // 1. merge the block's rows (8 per wave) into LDS
  for (int i = 0; i < UV_M / 4; ++i) {
    const int ml = w * (UV_M / 4) + i;
    const int m = mb * UV_M + ml;
    float acc[8];
    float lse = -INFINITY;
    if (m < m_total && nt > 0) {
      const int b = m / a.q_len, j = m % a.q_len;
      const int jh = j * a.n_heads + h;
      int first, count;
      unit_slots(a, nt, b, jh / kRowsPerWG, lane, first, count);
      lse = merge_row(a, first, count, jh % kRowsPerWG, lane, acc);
    }
    if (lse == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    }
    *(u32x4*)&s_o[ml][lane * 8] = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                        pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    if (a.lse != nullptr && lane == 0 && m < m_total)
      a.lse[(int64_t)m * a.n_heads + h] = lse;
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
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
  const int h = blockIdx.x / nmb;
  const int mb = blockIdx.x % nmb;
  const int m_total = a.batch * a.q_len;
  const int64_t nt = plan_total_tiles(a.seqlens, a.batch, a.row_groups, lane);
  for (int i = 0; i < UV_M / 4; ++i) {
    const int ml = w * (UV_M / 4) + i;
    const int m = mb * UV_M + ml;
    float acc[8];
    float lse = -INFINITY;
    if (m < m_total && nt > 0) {
      const int b = m / a.q_len, j = m % a.q_len;
      const int jh = j * a.n_heads + h;
      int first, count;
      unit_slots(a, nt, b, jh / kRowsPerWG, lane, first, count);
      lse = merge_row(a, first, count, jh % kRowsPerWG, lane, acc);
    }
    if (lse == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    }
    if (lane * 8 < a.d_lat) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[ml][lane * 8 + e] = acc[e];
    }
    if (a.lse != nullptr && lane == 0 && m < m_total)
      a.lse[(int64_t)m * a.n_heads + h] = lse;
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
    hipLaunchKernelGGL(combine_latent_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
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
