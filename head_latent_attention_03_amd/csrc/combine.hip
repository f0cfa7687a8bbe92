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
  const int64_t u = (int64_t)b * a.row_groups + rg;
  const int len = a.seqlens[b];
  const int f = a.unit_chunks[2 * u];
  const int c = a.unit_chunks[2 * u + 1];
  first = len > 0 ? f : 0;
  count = len > 0 ? c : 0;
}

// Merge the slice [W sl, W sl + W) of one row's partials (one thread).
// Partials are bf16 when the activations are bf16 and f32 otherwise.  The
// splits are taken in groups of 4 whose log-sum-exps and slices are loaded
// together, with a running maximum (the accumulated sum is rescaled when a
// group raises it), so the merge waits for one round of loads per group.
// Returns the row's log-sum-exp (-inf: no visible key, acc = 0).
constexpr int PART_GROUP = 4;

template <int W>
__device__ __forceinline__ void load_slice(const CombineArgs& a, int64_t slot, int r, int sl,
                                           float (&v)[W]) {
  if (a.out_dtype == DT_BF16) {
    const uint16_t* src = (const uint16_t*)a.part_o + (slot * kRowsPerWG + r) * a.d_lat + sl * W;
#pragma unroll
    for (int c = 0; c < W / 8; ++c) {
      const u32x4 u = *(const u32x4*)(src + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[c * 8 + 2 * e] = __uint_as_float(u[e] << 16);
        v[c * 8 + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
  } else {
    const float* src = (const float*)a.part_o + (slot * kRowsPerWG + r) * a.d_lat + sl * W;
#pragma unroll
    for (int c = 0; c < W / 4; ++c) {
      const f32x4 u = *(const f32x4*)(src + c * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[c * 4 + e] = u[e];
    }
  }
}

template <int W>
__device__ __forceinline__ float merge_slice(const CombineArgs& a, int first, int count, int r,
                                             int sl, float (&acc)[W]) {
#pragma unroll
  for (int e = 0; e < W; ++e) acc[e] = 0.f;
  float mx = -INFINITY, tot = 0.f;
  for (int s0 = 0; s0 < count; s0 += PART_GROUP) {
    float ls[PART_GROUP];
    float v[PART_GROUP][W];
#pragma unroll
    for (int s = 0; s < PART_GROUP; ++s) {
      const bool in = s0 + s < count;
      const int64_t slot = first + (in ? s0 + s : 0);
      ls[s] = in ? a.part_lse[slot * kRowsPerWG + r] : -INFINITY;
      load_slice<W>(a, slot, r, sl, v[s]);
    }
    float gm = ls[0];
#pragma unroll
    for (int s = 1; s < PART_GROUP; ++s) gm = fmaxf(gm, ls[s]);
    if (gm > mx) {
      // a new maximum: rescale what has been summed so far (0 on the first group)
      const float c = __expf(mx - gm);
      tot *= c;
#pragma unroll
      for (int e = 0; e < W; ++e) acc[e] *= c;
      mx = gm;
    }
#pragma unroll
    for (int s = 0; s < PART_GROUP; ++s) {
      // a split with no visible key (or past the count) weighs exactly 0
      const float wgt = ls[s] == -INFINITY ? 0.f : __expf(ls[s] - mx);
      tot += wgt;
#pragma unroll
      for (int e = 0; e < W; ++e) acc[e] += wgt == 0.f ? 0.f : wgt * v[s][e];
    }
  }
  if (mx == -INFINITY) return -INFINITY;
  const float inv = 1.0f / tot;
#pragma unroll
  for (int e = 0; e < W; ++e) acc[e] *= inv;
  return mx + __logf(tot);
}

// out = o~ (latent output): a workgroup merges 32 rows, thread = (row, slice
// of LAT_SLICE dims), 512 threads.  LAT_SLICE is 32 for the bf16 path
// (d_lat = 512) and 16 for the f32 path (d_lat a multiple of 16 up to 128),
// so every slice lies inside the row.
constexpr int ROWS_PER_WG = 32;

template <int LAT_SLICE>
__global__ __launch_bounds__(512) void combine_latent_kernel(CombineArgs a) {
  const int per_row = 512 / ROWS_PER_WG;       // slices per row (16)
  const int ml = threadIdx.x / per_row, sl = threadIdx.x % per_row;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_WG + ml;
  const int64_t rows = (int64_t)a.batch * a.q_len * a.n_heads;
  if (row >= rows || sl * LAT_SLICE >= a.d_lat) return;
  const int b = (int)(row / ((int64_t)a.q_len * a.n_heads));
  const int jh = (int)(row % ((int64_t)a.q_len * a.n_heads));
  int first, count;
  unit_slots(a, b, jh / kRowsPerWG, first, count);
  float acc[LAT_SLICE];
  const float lse = merge_slice<LAT_SLICE>(a, first, count, jh % kRowsPerWG, sl, acc);
  if (a.out_dtype == DT_BF16) {
    uint16_t* o = (uint16_t*)a.out + row * a.d_lat + sl * LAT_SLICE;
#pragma unroll
    for (int c = 0; c < LAT_SLICE / 8; ++c)
      *(u32x4*)(o + c * 8) = u32x4{pack_bf16x2(acc[c * 8], acc[c * 8 + 1]),
                                   pack_bf16x2(acc[c * 8 + 2], acc[c * 8 + 3]),
                                   pack_bf16x2(acc[c * 8 + 4], acc[c * 8 + 5]),
                                   pack_bf16x2(acc[c * 8 + 6], acc[c * 8 + 7])};
  } else {
    float* o = (float*)a.out + row * a.d_lat + sl * LAT_SLICE;
#pragma unroll
    for (int c = 0; c < LAT_SLICE / 4; ++c)
      *(f32x4*)(o + c * 4) = f32x4{acc[c * 4], acc[c * 4 + 1], acc[c * 4 + 2], acc[c * 4 + 3]};
  }
  if (a.lse != nullptr && sl == 0) a.lse[row] = lse;
}

// bf16: out[m, h, :] = W_UV[h] o~[m, h, :] for a block of 32 rows m = (b, j)
// of one head, 8 waves.  Each wave first issues the loads of its W_UV
// operands (16 rows n, all 512 k), which then stream in while the workgroup
// merges its rows (thread = (row, 32-dim slice)) into LDS as bf16.  The
// product runs on v_mfma_f32_16x16x32_bf16 as D^T = W_UV[h] o~^T: A = W rows
// (registers), B = o~ rows (LDS).
constexpr int UV_M = 32;
constexpr int UV_DLAT = 512;
constexpr int UV_DV = 128;
constexpr int UV_SLICE = 32;
constexpr int UV_PITCH = UV_DLAT + 8;        // bf16 elements per LDS row

__global__ __launch_bounds__(512) void combine_uv_bf16_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_o[UV_M][UV_PITCH];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
  // blocks of one head are adjacent in the logical order (shared W_UV in L2)
  const int blk = xcd_logical_id(blockIdx.x, gridDim.x);
  const int h = blk / nmb;
  const int mb = blk % nmb;
  const int m_total = a.batch * a.q_len;

  // 0. this wave's A operands: W_UV[h] rows n = 16w + lr, k = 32kk + 8lg ..
  const uint16_t* W = (const uint16_t*)a.w_uv + (int64_t)h * UV_DV * UV_DLAT;
  u16x8 wa[UV_DLAT / 32];
#pragma unroll
  for (int kk = 0; kk < UV_DLAT / 32; ++kk)
    wa[kk] = *(const u16x8*)(W + (int64_t)(w * 16 + lr) * UV_DLAT + kk * 32 + lg * 8);

  // 1. merge the block's rows into LDS: thread = (row, 32-dim slice)
  {
    const int ml = threadIdx.x / (UV_DLAT / UV_SLICE), sl = threadIdx.x % (UV_DLAT / UV_SLICE);
    const int m = mb * UV_M + ml;
    float acc[UV_SLICE];
    float lse = -INFINITY;
    if (m < m_total) {
      const int b = m / a.q_len, j = m % a.q_len;
      const int jh = j * a.n_heads + h;
      int first, count;
      unit_slots(a, b, jh / kRowsPerWG, first, count);
      lse = merge_slice<UV_SLICE>(a, first, count, jh % kRowsPerWG, sl, acc);
    } else {
#pragma unroll
      for (int e = 0; e < UV_SLICE; ++e) acc[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < UV_SLICE / 8; ++c)
      *(u32x4*)&s_o[ml][sl * UV_SLICE + c * 8] =
          u32x4{pack_bf16x2(acc[c * 8], acc[c * 8 + 1]), pack_bf16x2(acc[c * 8 + 2], acc[c * 8 + 3]),
                pack_bf16x2(acc[c * 8 + 4], acc[c * 8 + 5]), pack_bf16x2(acc[c * 8 + 6], acc[c * 8 + 7])};
    if (a.lse != nullptr && sl == 0 && m < m_total) a.lse[(int64_t)m * a.n_heads + h] = lse;
  }
  __syncthreads();

  // 2. D^T[n, m] = sum_k W[h, n, k] o~[m, k]; wave w: n block w, m blocks 0, 1
  f32x4 acc[2];
#pragma unroll
  for (int y = 0; y < 2; ++y) acc[y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < UV_DLAT / 32; ++kk) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const u16x8 ob = *(const u16x8*)&s_o[y * 16 + lr][kk * 32 + lg * 8];
      acc[y] = mfma_bf16_16x16x32(wa[kk], ob, acc[y]);
    }
  }
  // lane holds D^T[n = 16w + lg*4 + r][m = mblk*16 + lr]
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int m = mb * UV_M + y * 16 + lr;
    if (m >= m_total) continue;
    const int n0 = w * 16 + lg * 4;
    uint16_t* o = (uint16_t*)a.out + ((int64_t)m * a.n_heads + h) * UV_DV + n0;
    *(u32x2*)o = u32x2{pack_bf16x2(acc[y][0], acc[y][1]), pack_bf16x2(acc[y][2], acc[y][3])};
  }
}

// f32 (small shapes: d_lat <= 512, d_v <= 128): one workgroup per (head, 32 rows),
// merged rows in LDS, plain fp32 FMAs.
__global__ __launch_bounds__(256) void combine_uv_f32_kernel(CombineArgs a) {
  constexpr int SL = 16;                       // 8 slices of 16 cover d_lat <= 128
  __shared__ float s_o[UV_M][UV_DLAT + 4];
  const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
  const int h = blockIdx.x / nmb;
  const int mb = blockIdx.x % nmb;
  const int m_total = a.batch * a.q_len;
  {
    const int ml = threadIdx.x / 8, sl = threadIdx.x % 8;
    const int m = mb * UV_M + ml;
    if (sl * SL < a.d_lat) {
      float acc[SL];
      float lse = -INFINITY;
      if (m < m_total) {
        const int b = m / a.q_len, j = m % a.q_len;
        const int jh = j * a.n_heads + h;
        int first, count;
        unit_slots(a, b, jh / kRowsPerWG, first, count);
        lse = merge_slice<SL>(a, first, count, jh % kRowsPerWG, sl, acc);
      } else {
#pragma unroll
        for (int e = 0; e < SL; ++e) acc[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < SL; ++e) s_o[ml][sl * SL + e] = acc[e];
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
    const dim3 grid((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG));
    if (a.out_dtype == DT_BF16)
      hipLaunchKernelGGL(combine_latent_kernel<32>, grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(combine_latent_kernel<16>, grid, dim3(512), 0, s, a);
  } else {
    const int nmb = (a.batch * a.q_len + UV_M - 1) / UV_M;
    const unsigned grid = (unsigned)(nmb * a.n_heads);
    if (a.out_dtype == DT_BF16)
      hipLaunchKernelGGL(combine_uv_bf16_kernel, dim3(grid), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(combine_uv_f32_kernel, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
