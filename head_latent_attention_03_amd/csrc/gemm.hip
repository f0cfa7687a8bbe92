// Dense bf16 products around the MLA attention layer, gfx950: the latent
// down-projections of the hidden state and the weight-level absorption of
// W^UK into the query weights and of W^UV into the output projection
// ("Multi-Head Latent Attention: Scaling LLM Serving Throughput via Low-Rank
// KV Compression", section "Empirical Gains", the paragraph on absorbing
// W^UK into W^Q and W^UV into W^O; "Multi-Head Latent Attention – Latent
// KV-Cache (DeepSeek v3)", "Operation Flow", steps 1-2: the compressed
// latents come from the hidden state, the query parts from its latent).
//
//   gemm_nt_kernel   C[b, m, n] = sum_k A[b, m, k] B[b, n, k]   (bf16 in, fp32
//                    accumulate, bf16 or f32 out), on v_mfma_f32_32x32x16_bf16:
//                    workgroup = 128 x 128 outputs, 4 waves of 64 x 64 (2 x 2
//                    blocks of 32 x 32), k in chunks of 64 staged in LDS with
//                    16-byte rows padded to 144 bytes (conflict-free 16-byte
//                    reads); the next chunk's loads are issued before the
//                    current chunk's MFMAs.
//   gemm_nt_wide_kernel the same product for large m: workgroup = 256 x 160
//                    outputs, 4 waves of 64 x 160 (2 x 5 blocks of 32 x 32,
//                    accumulators in the accumulation registers), one
//                    workgroup per CU.  Ten MFMAs per seven 16-byte operand
//                    reads (against four per four), and a 4096 x 2112 output
//                    is 16 x 14 = 224 tiles, one round over 256 CUs, where
//                    128 x 128 tiles make 544 for 512 slots.
//   transpose_kernel dst[b, c, r] = src[b, r, c] for 16-bit elements, through
//                    a padded 32 x 32 LDS tile.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int GM = 128, GN = 128, GK = 64;
constexpr int GPITCH = GK * 2 + 16;   // bytes per staged row
constexpr int GTILE = GM * GPITCH;

__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][GTILE];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][GTILE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, lc = lane & 31;
  const int m0 = blockIdx.x * GM, n0 = blockIdx.y * GN, b = blockIdx.z;
  const uint8_t* A = (const uint8_t*)g.a + (int64_t)b * g.stride_a * 2;
  const uint8_t* Bm = (const uint8_t*)g.b + (int64_t)b * g.stride_b * 2;

  // this thread's 4 pieces (16 bytes) of each operand tile per k-chunk:
  // row = idx >> 3, piece = idx & 7, idx = tid + 256 e; rows past the matrix
  // read row 0 (their products are never stored)
  const uint8_t* ar[4];
  const uint8_t* br[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 256 * e, row = idx >> 3, pc = idx & 7;
    const int ma = m0 + row < g.m ? m0 + row : 0;
    const int nb = n0 + row < g.n ? n0 + row : 0;
    ar[e] = A + ((int64_t)ma * g.lda + pc * 8) * 2;
    br[e] = Bm + ((int64_t)nb * g.ldb + pc * 8) * 2;
  }
  u32x4 ra[4], rb[4];
  auto load = [&](int kc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pc = (tid + 256 * e) & 7;
      const bool in = kc * GK + pc * 8 < g.k;   // (k is a multiple of 8)
      ra[e] = in ? *(const u32x4*)(ar[e] + kc * GK * 2) : u32x4{0, 0, 0, 0};
      rb[e] = in ? *(const u32x4*)(br[e] + kc * GK * 2) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e, row = idx >> 3, pc = idx & 7;
      *(u32x4*)(&s_a[buf][row * GPITCH + pc * 16]) = ra[e];
      *(u32x4*)(&s_b[buf][row * GPITCH + pc * 16]) = rb[e];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int mr = 64 * (w >> 1), nc = 64 * (w & 1);
  const int nkc = (g.k + GK - 1) / GK;
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nkc) load(kc + 1);
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      u16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = *(const u16x8*)(&s_a[buf][(mr + 32 * i + lc) * GPITCH + (ks * 16 + 8 * hh) * 2]);
        bv[i] = *(const u16x8*)(&s_b[buf][(nc + 32 * i + lc) * GPITCH + (ks * 16 + 8 * hh) * 2]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
    }
    if (kc + 1 < nkc) {
      store(buf ^ 1);   // (the other buffer was last read before the barrier below)
      __syncthreads();
    }
  }
  // lane holds rows 8(r >> 2) + 4hh + (r & 3) of each 32-row block, column lc
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + mr + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m >= g.m) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + nc + 32 * j + lc;
        if (n >= g.n) continue;
        const int64_t o = (int64_t)b * g.stride_c + (int64_t)m * g.ldc + n;
        if (g.c_f32)
          ((float*)g.c)[o] = acc[i][j][r];
        else
          ((uint16_t*)g.c)[o] = (uint16_t)(pack_bf16x2(acc[i][j][r], 0.f) & 0xffffu);
      }
    }
}

constexpr int WM = 256, WN = 160;
constexpr int WTILE_A = WM * GPITCH, WTILE_B = WN * GPITCH;

// Grid (m blocks, n blocks, batch): consecutive workgroups go to consecutive
// XCDs, so with an m-block count that is a multiple of 8 every n block of an
// m block shares one XCD's L2 and its A rows are read from HBM once.
__global__ __launch_bounds__(256, 1) void gemm_nt_wide_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][WTILE_A];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][WTILE_B];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, lc = lane & 31;
  const int m0 = blockIdx.x * WM, n0 = blockIdx.y * WN, b = blockIdx.z;
  const uint8_t* A = (const uint8_t*)g.a + (int64_t)b * g.stride_a * 2;
  const uint8_t* Bm = (const uint8_t*)g.b + (int64_t)b * g.stride_b * 2;

  // 16-byte piece pc = tid & 7 of rows (tid >> 3) + 32 e: 8 rows of A and 5
  // of B per thread and k-chunk; rows past the matrix read row 0 (their
  // products are never stored)
  const int pc = tid & 7, r0 = tid >> 3;
  const uint8_t* ar[8];
  const uint8_t* br[5];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = m0 + r0 + 32 * e;
    ar[e] = A + ((int64_t)(row < g.m ? row : 0) * g.lda + pc * 8) * 2;
  }
#pragma unroll
  for (int e = 0; e < 5; ++e) {
    const int row = n0 + r0 + 32 * e;
    br[e] = Bm + ((int64_t)(row < g.n ? row : 0) * g.ldb + pc * 8) * 2;
  }
  // two register sets: chunk c is staged in set c & 1, so loads are issued
  // two chunks ahead of the MFMAs that use them
  u32x4 ra0[8], rb0[5], ra1[8], rb1[5];
  auto load = [&](int kc, u32x4 (&ra)[8], u32x4 (&rb)[5]) {
    const bool in = kc * GK + pc * 8 < g.k;   // (k is a multiple of 8)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      ra[e] = in ? *(const u32x4*)(ar[e] + kc * GK * 2) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 5; ++e)
      rb[e] = in ? *(const u32x4*)(br[e] + kc * GK * 2) : u32x4{0, 0, 0, 0};
  };
  auto store = [&](int buf, const u32x4 (&ra)[8], const u32x4 (&rb)[5]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *(u32x4*)(&s_a[buf][(r0 + 32 * e) * GPITCH + pc * 16]) = ra[e];
#pragma unroll
    for (int e = 0; e < 5; ++e)
      *(u32x4*)(&s_b[buf][(r0 + 32 * e) * GPITCH + pc * 16]) = rb[e];
  };
  f32x16 acc[2][5];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 5; ++j) acc[i][j] = f32x16{};
  const int mr = 64 * w;
  const int nkc = (g.k + GK - 1) / GK;
  // one chunk: MFMAs on LDS buffer kc & 1, then chunk kc + 1 from its set into
  // the other buffer (last read before the previous barrier) and chunk kc + 3
  // into the set just emptied
  auto step = [&](int kc, u32x4 (&ra)[8], u32x4 (&rb)[5]) {
    const int buf = kc & 1;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      u16x8 av[2], bv[5];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *(const u16x8*)(&s_a[buf][(mr + 32 * i + lc) * GPITCH + (ks * 16 + 8 * hh) * 2]);
#pragma unroll
      for (int j = 0; j < 5; ++j)
        bv[j] = *(const u16x8*)(&s_b[buf][(32 * j + lc) * GPITCH + (ks * 16 + 8 * hh) * 2]);
#pragma unroll
      for (int j = 0; j < 5; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
    }
    if (kc + 1 < nkc) {
      store(buf ^ 1, ra, rb);
      if (kc + 3 < nkc) load(kc + 3, ra, rb);
      __syncthreads();
    }
  };
  load(0, ra0, rb0);
  store(0, ra0, rb0);
  if (nkc > 1) load(1, ra1, rb1);
  if (nkc > 2) load(2, ra0, rb0);
  __syncthreads();
  for (int kc = 0; kc < nkc; kc += 2) {
    step(kc, ra1, rb1);   // stores chunk kc + 1 (odd: set 1)
    if (kc + 1 < nkc) step(kc + 1, ra0, rb0);
  }
  // lane holds rows 8(r >> 2) + 4hh + (r & 3) of each 32-row block, column lc
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + mr + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m >= g.m) continue;
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const int n = n0 + 32 * j + lc;
        if (n >= g.n) continue;
        const int64_t o = (int64_t)b * g.stride_c + (int64_t)m * g.ldc + n;
        if (g.c_f32)
          ((float*)g.c)[o] = acc[i][j][r];
        else
          ((uint16_t*)g.c)[o] = (uint16_t)(pack_bf16x2(acc[i][j][r], 0.f) & 0xffffu);
      }
    }
}

constexpr int TT = 32;

__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs t) {
  __shared__ uint16_t s[TT][TT + 2];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * TT, c0 = blockIdx.x * TT;
  const uint16_t* src = (const uint16_t*)t.src + (int64_t)b * t.rows * t.cols;
  uint16_t* dst = (uint16_t*)t.dst + (int64_t)b * t.rows * t.cols;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
#pragma unroll
  for (int k = 0; k < TT; k += 8) {
    const int r = r0 + ty + k, c = c0 + tx;
    if (r < t.rows && c < t.cols) s[ty + k][tx] = src[(int64_t)r * t.cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < TT; k += 8) {
    const int c = c0 + ty + k, r = r0 + tx;
    if (r < t.rows && c < t.cols) dst[(int64_t)c * t.rows + r] = s[tx][ty + k];
  }
}

// q_pe[m, h, :] = R(pos_m) q_rope[m, h, :] in fp32 (the rotation of the
// absorb kernel, for a query whose latent part came from absorbed weights):
// thread = one adjacent pair (x_2i, x_2i+1) of one (m, h) row; m = (b, j),
// pos_m = seqlens[b] - q_len + j.  In place is allowed.
__global__ __launch_bounds__(256) void rope_query_kernel(RopeArgs r) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int pairs = r.d_rope / 2;
  const int64_t total = (int64_t)r.batch * r.q_len * r.n_heads * pairs;
  if (idx >= total) return;
  const int i = (int)(idx % pairs);
  const int64_t row = idx / pairs;                  // (m, h)
  const int64_t m = row / r.n_heads;
  const int b = (int)(m / r.q_len), j = (int)(m % r.q_len);
  const int pos = r.seqlens[b] - r.q_len + j;
  const uint32_t x = *(const uint32_t*)((const uint16_t*)r.src + row * r.d_rope + 2 * i);
  float y0, y1;
  rope_pair(bf16_bits_to_f32((uint16_t)(x & 0xffffu)), bf16_bits_to_f32((uint16_t)(x >> 16)),
            pos, rope_theta(i, r.d_rope, r.rope_base), y0, y1);
  *(uint32_t*)((uint16_t*)r.dst + row * r.d_rope + 2 * i) = pack_bf16x2(y0, y1);
}

}  // namespace

hipError_t launch_rope_query(const RopeArgs& r, hipStream_t s) {
  const int64_t total = (int64_t)r.batch * r.q_len * r.n_heads * (r.d_rope / 2);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_query_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, r);
  return hipGetLastError();
}

bool gemm_nt_takes_wide_tiles(const GemmArgs& g) {
  // the wide tile when there are at least 512 rows and at least half a round
  // of its tiles over the 256 CUs; smaller products keep the 128 x 128 tile,
  // whose smaller waste on ragged edges and two workgroups per CU win there
  const int64_t tiles = ((int64_t)(g.m + WM - 1) / WM) * ((g.n + WN - 1) / WN) * g.batch;
  return g.m >= 512 && tiles >= 128;
}

hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t s) {
  if (gemm_nt_takes_wide_tiles(g)) {
    const dim3 grid((g.m + WM - 1) / WM, (g.n + WN - 1) / WN, g.batch);
    hipLaunchKernelGGL(gemm_nt_wide_kernel, grid, dim3(256), 0, s, g);
    return hipGetLastError();
  }
  const dim3 grid((g.m + GM - 1) / GM, (g.n + GN - 1) / GN, g.batch);
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& t, hipStream_t s) {
  const dim3 grid((t.cols + TT - 1) / TT, (t.rows + TT - 1) / TT, t.batch);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, t);
  return hipGetLastError();
}

}  // namespace mla
