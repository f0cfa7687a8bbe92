// Query absorption and rotary embedding of the decoupled query, gfx950.
//
//   q~[m, h, :]  = W_UK[h]^T q^C[m, h, :]      (W^UK absorbed into the query
//                  side: "Multi-Head Latent Attention: Scaling LLM Serving
//                  Throughput via Low-Rank KV Compression", section "Empirical
//                  Gains", paragraph on absorption)
//   q_pe[m, h, :] = R(pos_m) q^R[m, h, :]      (decoupled RoPE, same section;
//                  adjacent pairs (x_2i, x_2i+1) rotated by pos * base^(-2i/d_R)
//                  as on the rotary page "Deepseek-V3 Define 1: Higher
//                  Attachment of Head", in FP32 as "Multi-Head Latent Attention
//                  – Latent KV-Cache (DeepSeek v3)" prescribes for RoPE)
// where m = (b, j) and pos_m = seqlens[b] - q_len + j.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

// ---------------------------------------------------------------------------
// bf16 (d_nope = 128, d_lat = 512): one workgroup per (head h, NB latent
// columns, M rows m).  The W_UK[h] slice [128 x NB] bf16 is staged in LDS and
// read as the A operand of D^T = W_UK[h]^T q^C^T with the LDS transpose read;
// q^C rows are the B operand straight from global memory.  NB = 256, M = 64
// for bf16 output (2 column blocks per head: at 128 heads one workgroup per
// CU); NB = 512, M = 32 for e4m3 output, whose per-row scale max|q~| / 448
// needs the whole row in one workgroup (two row blocks per head for 64 rows).
constexpr int AB_M = 64;
constexpr int AB_K = 128;    // d_nope
constexpr int AB_N = 512;    // d_lat
constexpr int AB_ROPE = 64;  // d_rope

template <int NB, bool FP8, int M>
__global__ __launch_bounds__(256, 1) void absorb_bf16_kernel(AbsorbArgs a) {
  // row pitch NB*2 + 32 bytes: the four rows of a transpose-read group land
  // on disjoint banks
  constexpr int PITCH = NB * 2 + 32;
  constexpr int NBLK = NB / 16 / 4;            // 16-column blocks per wave
  constexpr int NY = M / 16;                    // 16-row blocks
  __shared__ __attribute__((aligned(16))) uint8_t s_w[AB_K * PITCH];
  __shared__ float s_amax[4][M];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int nmb = (a.batch * a.q_len + M - 1) / M;
  constexpr int NCB = AB_N / NB;               // column blocks per head
  const int blk = xcd_logical_id(blockIdx.x, gridDim.x);
  const int h = blk / (nmb * NCB);
  const int cb = (blk / nmb) % NCB;
  const int mb = blk % nmb;
  const int m_total = a.batch * a.q_len;

  // every global load of the workgroup is issued before the first use:
  // the W_UK[h][:, cb*NB .. +NB] slice (row k = content coordinate), the q^C
  // rows (B operand) and this block's share of the rotary rows
  const uint16_t* W = (const uint16_t*)a.w_uk + (int64_t)h * AB_K * AB_N + cb * NB;
  constexpr int CHUNKS = AB_K * NB / 8;        // 16-byte chunks
  constexpr int PER_T = CHUNKS / 256;
  u32x4 stage[PER_T];
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    const int c = threadIdx.x + i * 256;
    const int row = c / (NB / 8), col = c % (NB / 8);
    stage[i] = *(const u32x4*)&W[(int64_t)row * AB_N + col * 8];
  }
  // B operand: q^C rows (m = lr within 16-row block y), k = kk*32 + lg*8 ..
  u16x8 qb[NY][AB_K / 32];
#pragma unroll
  for (int y = 0; y < NY; ++y) {
    const int m = mb * M + y * 16 + lr;
    const bool valid = m < m_total;
    const uint16_t* q = (const uint16_t*)a.q_nope + ((int64_t)(valid ? m : 0) * a.n_heads + h) * AB_K;
#pragma unroll
    for (int kk = 0; kk < AB_K / 32; ++kk) {
      const u16x8 v = *(const u16x8*)(q + kk * 32 + lg * 8);
      qb[y][kk] = valid ? v : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // rotary part: the NCB column blocks of a head split its M rows; thread t
  // rotates pair t % 32 of rows (t + 256 e) / 32 of this block's share
  constexpr int PAIRS = AB_ROPE / 2;
  constexpr int RROWS = M / NCB;
  constexpr int RPER = (RROWS * PAIRS + 255) / 256;
  uint32_t rq[RPER];
  int rpos[RPER];
  bool rvalid[RPER];
#pragma unroll
  for (int e = 0; e < RPER; ++e) {
    const int idx = threadIdx.x + e * 256;
    const int m = mb * M + cb * RROWS + idx / PAIRS;
    const bool valid = idx < RROWS * PAIRS && m < m_total;
    const int mm = valid ? m : 0;
    const int64_t off = ((int64_t)mm * a.n_heads + h) * AB_ROPE + 2 * (idx % PAIRS);
    rq[e] = *(const uint32_t*)((const uint16_t*)a.q_rope + off);
    // (a position may be negative when a sequence holds fewer than q_len tokens)
    rpos[e] = a.seqlens[mm / a.q_len] - a.q_len + mm % a.q_len;
    rvalid[e] = valid;
  }
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    const int c = threadIdx.x + i * 256;
    const int row = c / (NB / 8), col = c % (NB / 8);
    *(u32x4*)&s_w[row * PITCH + col * 16] = stage[i];
  }
  {
    const double theta = rope_theta(threadIdx.x % PAIRS, AB_ROPE, a.rope_base);
#pragma unroll
    for (int e = 0; e < RPER; ++e) {
      if (!rvalid[e]) continue;
      const int idx = threadIdx.x + e * 256;
      const int m = mb * M + cb * RROWS + idx / PAIRS;
      const int64_t off = ((int64_t)m * a.n_heads + h) * AB_ROPE + 2 * (idx % PAIRS);
      float y0, y1;
      rope_pair(__uint_as_float(rq[e] << 16), __uint_as_float(rq[e] & 0xffff0000u), rpos[e],
                theta, y0, y1);
      *(uint32_t*)((uint16_t*)a.q_pe + off) = pack_bf16x2(y0, y1);
    }
  }
  __syncthreads();

  // wave w: columns n in [w*NB/4, (w+1)*NB/4) of the block = NBLK blocks of 16
  f32x4 acc[NBLK][NY];
#pragma unroll
  for (int x = 0; x < NBLK; ++x)
#pragma unroll
    for (int y = 0; y < NY; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < AB_K / 32; ++kk) {
#pragma unroll
    for (int x = 0; x < NBLK; ++x) {
      // A[m' = n][k] = W[k][n]: lane (lg, lr) addresses W row kk*32 + lg*8 + lr/4
      // (+4 for the second half), columns n0 + (lr&3)*4 .. +3
      const int n0 = (w * NBLK + x) * 16;
      const MLA_LDS uint8_t* p = (const MLA_LDS uint8_t*)s_w +
                                 (kk * 32 + lg * 8 + (lr >> 2)) * PITCH + (n0 + (lr & 3) * 4) * 2;
      const u16x4 lo = lds_read_tr16(p);
      const u16x4 hi = lds_read_tr16(p + 4 * PITCH);
      const u16x8 av = u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int y = 0; y < NY; ++y) acc[x][y] = mfma_bf16_16x16x32(av, qb[y][kk], acc[x][y]);
    }
  }
  // lane holds q~^T[n = cb*NB + n0 + lg*4 + r][m = y*16 + lr]
  if constexpr (!FP8) {
    // the rows go through LDS (the W slice is no longer needed) so that each
    // store writes 16 contiguous bytes per lane, whole rows per wave
    constexpr int OP = NB * 2 + 16;            // LDS pitch of a staged row
    static_assert(M * OP <= AB_K * PITCH, "the staged rows fit");
    __syncthreads();
#pragma unroll
    for (int y = 0; y < NY; ++y)
#pragma unroll
      for (int x = 0; x < NBLK; ++x) {
        const int n = (w * NBLK + x) * 16 + lg * 4;
        *(MLA_LDS u32x2*)((MLA_LDS uint8_t*)s_w + (y * 16 + lr) * OP + n * 2) =
            u32x2{pack_bf16x2(acc[x][y][0], acc[x][y][1]), pack_bf16x2(acc[x][y][2], acc[x][y][3])};
      }
    __syncthreads();
    constexpr int RC = NB / 8;                 // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < M * RC / 256; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int ml = c / RC, ch = c % RC;
      const int m = mb * M + ml;
      if (m < m_total)
        *(u32x4*)((uint16_t*)a.q_lat + ((int64_t)m * a.n_heads + h) * AB_N + cb * NB + ch * 8) =
            *(const MLA_LDS u32x4*)((const MLA_LDS uint8_t*)s_w + ml * OP + ch * 16);
    }
  } else {
    static_assert(NB == AB_N, "the e4m3 row scale needs the whole row");
    // row amax over all 512 columns: lanes -> waves -> LDS
#pragma unroll
    for (int y = 0; y < NY; ++y) {
      float mx = 0.f;
#pragma unroll
      for (int x = 0; x < NBLK; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[x][y][r]));
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      if (lg == 0) s_amax[w][y * 16 + lr] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int y = 0; y < NY; ++y) {
      const int ml = y * 16 + lr;
      const int m = mb * M + ml;
      const float amax = fmaxf(fmaxf(s_amax[0][ml], s_amax[1][ml]), fmaxf(s_amax[2][ml], s_amax[3][ml]));
      // the row scale is the smallest power of two with amax / scale <= 448,
      // so that the scaling itself is exact and the decode can apply it as
      // an MFMA block-scale exponent (an all-zero row takes 1)
      int ex = 0;
      if (amax > 0.f) {
        const float f = frexpf(amax * (1.0f / 448.0f), &ex);
        if (f == 0.5f) --ex;
        ex = min(max(ex, -126), 127);
      }
      const float sc = ldexpf(1.0f, ex);
      const float inv = ldexpf(1.0f, -ex);
      if (m >= m_total) continue;
      uint8_t* o = (uint8_t*)a.q_lat + ((int64_t)m * a.n_heads + h) * AB_N;
#pragma unroll
      for (int x = 0; x < NBLK; ++x) {
        const int n = (w * NBLK + x) * 16 + lg * 4;
        int pk = 0;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fminf(fmaxf(acc[x][y][r] * inv, -448.f), 448.f);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], pk, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
        *(int*)(o + n) = pk;
      }
      if (w == 0 && lg == 0) a.q_lat_scale[(int64_t)m * a.n_heads + h] = sc;
    }
  }
}

// ---------------------------------------------------------------------------
// f32 (small shapes): one thread per output element.
__global__ __launch_bounds__(256) void absorb_f32_kernel(AbsorbArgs a) {
  const int64_t total_lat = (int64_t)a.batch * a.q_len * a.n_heads * a.d_lat;
  const int64_t total_pe = (int64_t)a.batch * a.q_len * a.n_heads * (a.d_rope / 2);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < total_lat) {
    const int n = (int)(idx % a.d_lat);
    const int64_t mh = idx / a.d_lat;
    const int h = (int)(mh % a.n_heads);
    const float* q = (const float*)a.q_nope + mh * a.d_nope;
    const float* W = (const float*)a.w_uk + (int64_t)h * a.d_nope * a.d_lat + n;
    float s = 0.f;
    for (int k = 0; k < a.d_nope; ++k) s = fmaf(q[k], W[(int64_t)k * a.d_lat], s);
    ((float*)a.q_lat)[idx] = s;
  } else if (idx < total_lat + total_pe) {
    const int64_t p = idx - total_lat;
    const int i = (int)(p % (a.d_rope / 2));
    const int64_t mh = p / (a.d_rope / 2);
    const int64_t m = mh / a.n_heads;
    const int b = (int)(m / a.q_len), j = (int)(m % a.q_len);
    const int pos = a.seqlens[b] - a.q_len + j;
    const float* qr = (const float*)a.q_rope + mh * a.d_rope + 2 * i;
    float y0, y1;
    rope_pair(qr[0], qr[1], pos, rope_theta(i, a.d_rope, a.rope_base), y0, y1);
    float* o = (float*)a.q_pe + mh * a.d_rope + 2 * i;
    o[0] = y0;
    o[1] = y1;
  }
}

}  // namespace

hipError_t launch_absorb_bf16(const AbsorbArgs& a, bool fp8_out, hipStream_t s) {
  const int m_total = a.batch * a.q_len;
  if (m_total * a.n_heads == 0) return hipSuccess;
  if (fp8_out) {
    // the e4m3 row scale needs the whole 512-column row in one workgroup: 32
    // rows per workgroup keep the grid at two workgroups per head for 64 rows
    constexpr int M = 32;
    const int nmb = (m_total + M - 1) / M;
    hipLaunchKernelGGL((absorb_bf16_kernel<AB_N, true, M>), dim3((unsigned)(nmb * a.n_heads)),
                       dim3(256), 0, s, a);
  } else {
    constexpr int NB = 256, M = AB_M;
    const int nmb = (m_total + M - 1) / M;
    hipLaunchKernelGGL((absorb_bf16_kernel<NB, false, M>),
                       dim3((unsigned)(nmb * a.n_heads * (AB_N / NB))), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_absorb_f32(const AbsorbArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.q_len * a.n_heads * (a.d_lat + a.d_rope / 2);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(absorb_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
