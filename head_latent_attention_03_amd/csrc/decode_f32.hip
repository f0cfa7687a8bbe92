// Split-KV MLA decode, fp32 latent and activations, small head shapes
// (d_lat <= 128, d_rope <= 32), gfx950.
//
// Same computation, split plan and partial layout as the bf16 kernel (see
// decode_bf16.hip): s[t] = scale * (q~ . c_t + q_pe . k^R_t), softmax over
// the chunk's visible tokens, o~ = sum_t p_t c_t, written with its
// log-sum-exp.  Here one thread owns one (query, head) row and walks the
// chunk's tokens with plain fp32 FMAs and an ordinary online softmax; the
// tokens of a tile are read by all threads of the workgroup at once, so they
// come from L1/L2 after the first reader.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int DL_MAX = 128;
constexpr int DR_MAX = 32;

__global__ __launch_bounds__(128) void decode_f32_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  int g;
  Chunk ch;
  if (!plan_locate(a.seqlens, a.batch, a.row_groups, a.num_wg, blockIdx.x, lane, g, ch)) return;
  if (ch.c == 0 && threadIdx.x == 0) {
    // where the combine pass finds this unit's partials
    const int64_t u = (int64_t)ch.b * a.row_groups + ch.rg;
    a.unit_chunks[2 * u] = g;
    a.unit_chunks[2 * u + 1] = ch.splits;
  }
  const int k0 = (int)((int64_t)ch.c * ch.tiles / ch.splits);
  const int k1 = (int)((int64_t)(ch.c + 1) * ch.tiles / ch.splits);
  const int t_begin = k0 * kTile;
  const int t_end = min(k1 * kTile, ch.len);

  const int row = threadIdx.x;                        // 0..127
  const int R = ch.rg * kRowsPerWG + row;
  const bool valid = R < a.q_len * a.n_heads;
  const int j = valid ? R / a.n_heads : 0;
  const int h = valid ? R % a.n_heads : 0;
  const int lim = valid ? (a.causal ? ch.len - a.q_len + j + 1 : ch.len) : 0;
  const int64_t qrow = ((int64_t)ch.b * a.q_len + j) * a.n_heads + h;
  const float* ql = (const float*)a.q_lat + qrow * a.d_lat;
  const float* qp = (const float*)a.q_pe + qrow * a.d_rope;

  float q[DL_MAX], qr[DR_MAX], o[DL_MAX];
#pragma unroll
  for (int d = 0; d < DL_MAX; ++d) {
    q[d] = (valid && d < a.d_lat) ? ql[d] : 0.f;
    o[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < DR_MAX; ++d) qr[d] = (valid && d < a.d_rope) ? qp[d] : 0.f;

  const float* lat = (const float*)a.kv_lat;
  const float* rope = (const float*)a.kv_rope;
  const int32_t* bt = a.block_table + (int64_t)ch.b * a.max_pages;
  float m = -INFINITY, l = 0.f;
  const int t_stop = min(t_end, lim);
  for (int t = t_begin; t < t_stop; ++t) {
    const int64_t prow = (int64_t)bt[t / kPage] * kPage + (t % kPage);
    const float* c = lat + prow * a.d_lat;
    const float* kr = rope + prow * a.d_rope;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DL_MAX; ++d)
      if (d < a.d_lat) s = fmaf(q[d], c[d], s);
#pragma unroll
    for (int d = 0; d < DR_MAX; ++d)
      if (d < a.d_rope) s = fmaf(qr[d], kr[d], s);
    s *= a.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < DL_MAX; ++d)
      if (d < a.d_lat) o[d] = o[d] * alpha + p * c[d];
    m = m_new;
  }
  const int64_t slot = g;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  float* dst = (float*)a.part_o + (slot * kRowsPerWG + row) * a.d_lat;
#pragma unroll
  for (int d = 0; d < DL_MAX; ++d)
    if (d < a.d_lat) dst[d] = o[d] * inv;
  a.part_lse[slot * kRowsPerWG + row] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_f32_kernel, dim3(grid), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
