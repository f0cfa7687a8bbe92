// Non-absorbed MLA attention for many query tokens per sequence (chunked
// prefill, multi-token verification), gfx950, bf16.
//
// The same attention as the decode path, in the other of the two
// functionally equivalent forms ("Related papers: SnapMLA: Efficient
// Long-Context MLA Decoding via H…", the abstract on two kernel formulations
// of MLA; "Multi-Head Latent Attention: Scaling LLM Serving Throughput via
// Low-Rank KV Compression", section "Empirical Gains": keys and values come
// from the cached latent through W^UK and W^UV):
//   K^C[t, h] = W_UK[h] c_t,  V[t, h] = W_UV[h] c_t            (expand_kv_kernel)
//   s[j, t]   = scale ( q^C[j, h] . K^C[t, h] + R(pos_j) q^R[j, h] . k^R_t )
//   out[j, h] = sum_t softmax_t(s) V[t, h]   (causal: t <= pos_j)   (attn_kernel)
// Absorbing W_UK into the query costs 2 (d_c + d_R + d_c) flops per key and
// query row; expanding costs 2 d_c (d_nope + d_v) per key and head once, then
// 2 (d_nope + d_R + d_v) per key and query row, so with many query rows per
// sequence the expanded form does far less arithmetic.
//
// The expansion is a GEMM per sequence: [L_b x 512] (latent rows gathered
// through the block table) times [512 x 2 * 128 * n_heads] (the rows of W_UK
// and W_UV), on v_mfma_f32_32x32x16_bf16, written to the workspace as bf16
// K^C and V [B, H, L_pad, 128].  Expanding per key tile inside the attention
// kernel instead would stream W_UK[h] and W_UV[h] (256 KiB per head) through
// every workgroup for every tile, four times the tile's own bytes.
//
// The attention is flash attention with online softmax (running maximum and
// output rescale) per workgroup of 128 query rows of one (sequence, head):
// wave w owns rows 32w .. 32w+31.  S^T = K Q^T on 32x32x16 MFMAs (K rows
// from LDS, Q^T from registers), so each lane holds one query row and 16
// keys per 32-key block; O^T += V^T P^T with P^T straight from the score
// registers and V^T read with the LDS transpose read in the same key order.
// Key tiles of 32 keep a workgroup small enough (registers and LDS) for two
// to share a CU.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int D_LAT = 512;
constexpr int D_NOPE = 128;
constexpr int D_V = 128;
constexpr int D_ROPE = 64;

// ---------------------------------------------------------------------------
// expansion GEMM: workgroup = (head h, half p: K^C or V, sequence b, slice of
// its tokens).  Wave w keeps rows n = 32w .. 32w+31 of W_UK[h] (p = 0) or
// W_UV[h] (p = 1), all 512 k, in 128 registers as the A operand of
// D^T = W c^T, and the latent streams past them through a ring of EX_NS
// stages of 32 tokens, copied straight from HBM into LDS EX_AHEAD tiles
// ahead.  Two workgroups share a CU, so one's MFMAs run while the other waits.
// Chunk c of token row r's 1 KiB sits at slot c ^ (r & 15) of the row, so
// that the 16 lanes of a 16-byte read (rows r .. r + 15, one chunk) fall on 16
// different bank groups.  A 32-token tile lies inside one 64-token page (its
// rows past the sequence end re-read the last token, which lies in the same
// page); the slice's pages are read into LDS first, so that no vector load
// the compiler waits for sits among the copies.
constexpr int EX_T = 32;                       // tokens per tile
constexpr int EX_NS = 2;                       // ring stages
constexpr int EX_AHEAD = EX_NS - 1;            // tiles whose copies are in flight
constexpr int EX_OCC = 2;                      // workgroups per CU (64 KiB of LDS, 238 registers each)
constexpr int EX_ROW = D_LAT * 2;              // 1 KiB latent row
constexpr int EX_STAGE = EX_T * EX_ROW;        // 32 KiB
constexpr int EX_KS = D_LAT / 16;              // 32 MFMA k-steps
constexpr int EX_MAX_SLICE = 128;              // tiles per slice at most (4096 tokens)
constexpr int EX_RB = 4;                       // latent operand reads issued a group ahead

template <int N>
__device__ __forceinline__ void ex_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `later` tiles' copies (EX_T / 4 per wave each) are
// outstanding (later < EX_AHEAD)
template <int L = 0>
__device__ __forceinline__ void ex_wait_tiles(int later) {
  if constexpr (L < EX_AHEAD - 1) {
    if (later <= L) {
      ex_wait_vm<L * (EX_T / 4)>();
      return;
    }
    ex_wait_tiles<L + 1>(later);
  } else {
    ex_wait_vm<L * (EX_T / 4)>();
  }
}

__device__ __forceinline__ void ex_copy16(const void* sbase, uint32_t voff,
                                          const MLA_LDS uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

__global__ __launch_bounds__(256, EX_OCC) void expand_kv_kernel(PrefillArgs a, int slice_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lat[EX_NS][EX_STAGE];
  __shared__ int32_t s_page[EX_MAX_SLICE / 2 + 1];
  const int h = blockIdx.x >> 1, part = blockIdx.x & 1, b = blockIdx.y;
  const int len = a.seqlens[b];
  const int tile0 = blockIdx.z * slice_tiles;
  const int ntiles = min((len + EX_T - 1) / EX_T - tile0, slice_tiles);
  if (ntiles <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, lc = lane & 31;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  // pages of tiles tile0 .. tile0 + ntiles - 1 (two tiles per page; a slice
  // may start in the middle of a page)
  const int pg0 = tile0 * EX_T / kPage;
  const int npg = (tile0 + ntiles - 1) * EX_T / kPage - pg0 + 1;
  if (tid < npg) s_page[tid] = bt_row[pg0 + tid];
  __syncthreads();

  // tile kt's rows 8w .. 8w + 7 into stage st: lane l brings chunk l ^ (r & 15)
  // of row r (rows past the sequence re-read its last token, finite data whose
  // outputs are not stored)
  const uint8_t* lat = (const uint8_t*)a.kv_lat;
  // row r = 8w + j: r & 15 = 8 (w & 1) + j
  const uint32_t lane_key = (uint32_t)(lane ^ (8 * (w & 1)));
  auto copy_tile = [&](int kt, int st) {
    const uint8_t* pbase =
        lat + (int64_t)__builtin_amdgcn_readfirstlane(s_page[(tile0 + kt) * EX_T / kPage - pg0]) *
                  kPage * EX_ROW;
#pragma unroll
    for (int j = 0; j < EX_T / 4; ++j) {
      const int r = (EX_T / 4) * w + j;
      const int t = min((tile0 + kt) * EX_T + r, len - 1);
      ex_copy16(pbase + (int64_t)(t % kPage) * EX_ROW, (lane_key ^ (uint32_t)j) << 4,
                (MLA_LDS uint8_t*)s_lat[st] + r * EX_ROW);
    }
  };
#pragma unroll
  for (int kt = 0; kt < EX_AHEAD; ++kt)
    if (kt < ntiles) copy_tile(kt, kt);

  // A operands: W rows n = 32w + lc, k = 16 ks + 8 hh .. + 7
  u16x8 wr[EX_KS];
  {
    const uint16_t* pw = (const uint16_t*)(part ? a.w_uv : a.w_uk) +
                         ((int64_t)h * 128 + 32 * w + lc) * D_LAT + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < EX_KS; ++ks) wr[ks] = *(const u16x8*)(pw + 16 * ks);
  }
  // the compiler's wait for W (all older copies with it) happens here, once
#pragma unroll
  for (int ks = 0; ks < EX_KS; ++ks) asm volatile("" ::"v"(wr[ks]));

  uint16_t* dst = (uint16_t*)(part ? a.vexp : a.kexp) + ((int64_t)b * a.n_heads + h) * a.lpad * 128;
  for (int kt = 0; kt < ntiles; ++kt) {
    // tile kt's copies have landed (those of up to EX_AHEAD - 1 later tiles
    // may not)
    ex_wait_tiles(min(EX_AHEAD - 1, ntiles - 1 - kt));
    __syncthreads();
    // stage (kt + EX_AHEAD) % EX_NS held tile kt - 1, which every wave left
    // before the barrier
    if (kt + EX_AHEAD < ntiles) copy_tile(kt + EX_AHEAD, (kt + EX_AHEAD) % EX_NS);
    const MLA_LDS uint8_t* st = (const MLA_LDS uint8_t*)s_lat[kt % EX_NS] + lc * EX_ROW;
    // two accumulators (even and odd k-steps) so that consecutive MFMAs do not
    // wait on each other
    // The latent operands of k-steps k0 + EX_RB .. are read before the MFMAs of
    // k0 .. (scheduling barriers keep that order), so every read has EX_RB
    // MFMAs to land behind.
    f32x16 d0 = f32x16{}, d1 = f32x16{};
    auto read_group = [&](int k0, u16x8(&cb)[EX_RB]) {
#pragma unroll
      for (int e = 0; e < EX_RB; ++e) {
        const int c = 2 * (k0 + e) + hh;
        cb[e] = *(const MLA_LDS u16x8*)(st + ((c ^ (lc & 15)) << 4));
      }
    };
    u16x8 cur[EX_RB], nxt[EX_RB];
    read_group(0, cur);
#pragma unroll
    for (int k0 = 0; k0 < EX_KS; k0 += EX_RB) {
      __builtin_amdgcn_sched_barrier(0);
      if (k0 + EX_RB < EX_KS) read_group(k0 + EX_RB, nxt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < EX_RB; e += 2) {
        d0 = mfma32(wr[k0 + e], cur[e], d0);
        d1 = mfma32(wr[k0 + e + 1], cur[e + 1], d1);
      }
#pragma unroll
      for (int e = 0; e < EX_RB; ++e) cur[e] = nxt[e];
    }
    // lane: token lc of the tile, dims 32w + 8g + 4hh .. + 3 (g = 0..3)
    const int t = (tile0 + kt) * EX_T + lc;
    if (t < len) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t o = (int64_t)t * 128 + 32 * w + 8 * g + 4 * hh;
        *(u32x2*)(dst + o) =
            u32x2{pack_bf16x2(d0[4 * g] + d1[4 * g], d0[4 * g + 1] + d1[4 * g + 1]),
                  pack_bf16x2(d0[4 * g + 2] + d1[4 * g + 2], d0[4 * g + 3] + d1[4 * g + 3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// attention: workgroup = (128 query rows of sequence b, head h)
constexpr int QB = 128;                  // query rows per workgroup
constexpr int KT = 32;                   // keys per tile (half a cache page)
constexpr int NBK = KT / 32;             // 32-key MFMA blocks per tile
constexpr int NPK = KT * 16 / 256;       // 16-byte K^C (and V) pieces per thread and tile
constexpr int NPR = KT * 8 / 256;        // 16-byte rotary pieces per thread and tile
constexpr int ATT_OCC = 2;               // workgroups per CU (247 registers, 2 x 23.5 KiB of LDS each)
constexpr int K_PITCH = D_NOPE * 2 + 16; // 272: conflict-free 16-byte row reads
constexpr int R_PITCH = D_ROPE * 2 + 16; // 144
constexpr int V_PITCH = D_V * 2 + 64;    // 320: conflict-free transpose reads
constexpr int K_OFF = 0;
constexpr int R_OFF = KT * K_PITCH;
constexpr int V_OFF = R_OFF + KT * R_PITCH;
constexpr int STAGE = V_OFF + KT * V_PITCH;
constexpr int KS_N = D_NOPE / 16;        // 8 score k-steps over q^C
constexpr int KS = KS_N + D_ROPE / 16;   // 12
constexpr float kLazy = 8.f;             // log2 units a row maximum may pass m by

__global__ __launch_bounds__(256, ATT_OCC) void attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][STAGE];
  // the row blocks of one (sequence, head) take consecutive logical ids on one
  // XCD, so that its expanded K and V pass through one L2
  const int nrb = gridDim.x;
  const int nblk = nrb * gridDim.y * gridDim.z;
  const int lid = xcd_logical_id(blockIdx.x + nrb * (blockIdx.y + gridDim.y * blockIdx.z), nblk);
  const int b = lid / (nrb * gridDim.y), h = (lid / nrb) % gridDim.y;
  const int j0 = (lid % nrb) * QB;
  const int len = a.seqlens[b];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, lc = lane & 31;
  const int H = a.n_heads;
  // the lane's query row (j >= q_len: a padding row, masked throughout)
  const int j = j0 + 32 * w + lc;
  const bool row_ok = j < a.q_len;
  const int jr = row_ok ? j : 0;
  const int pos = len - a.q_len + j;         // the row sees keys t <= pos
  const int lim = row_ok ? min(pos + 1, len) : 0;
  // keys the workgroup needs: up to the last valid row's position
  const int jmax = min(j0 + QB, a.q_len) - 1;
  const int kend = max(0, min(len, len - a.q_len + jmax + 1));
  const int ntiles = (kend + KT - 1) / KT;

  // Q^T operand: dims 16ks + 8hh .. +7 of the lane's row; q^R rotated in fp32
  u16x8 q[KS];
  {
    const int64_t qrow = ((int64_t)b * a.q_len + jr) * H + h;
    const uint16_t* qn = (const uint16_t*)a.q_nope + qrow * D_NOPE;
    const uint16_t* qr = (const uint16_t*)a.q_rope + qrow * D_ROPE;
#pragma unroll
    for (int ks = 0; ks < KS_N; ++ks) q[ks] = *(const u16x8*)(qn + ks * 16 + hh * 8);
    const int p = max(pos, 0);
#pragma unroll
    for (int ks = KS_N; ks < KS; ++ks) {
      const int d0 = (ks - KS_N) * 16 + hh * 8;
      const u16x8 x = *(const u16x8*)(qr + d0);
      u16x8 y;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float y0, y1;
        rope_pair(bf16_bits_to_f32(x[e]), bf16_bits_to_f32(x[e + 1]), p,
                  rope_theta((d0 + e) / 2, D_ROPE, a.rope_base), y0, y1);
        const uint32_t pr = pack_bf16x2(y0, y1);
        y[e] = (uint16_t)(pr & 0xffffu);
        y[e + 1] = (uint16_t)(pr >> 16);
      }
      q[ks] = y;
    }
  }

  // tile loads, register staged two tiles ahead (two sets, so that a tile's
  // loads have the compute of two tiles to land in before they are stored
  // to LDS): K^C and V 4 pieces each, k^R 2 pieces
  const uint8_t* kx = (const uint8_t*)a.kexp + ((int64_t)b * H + h) * a.lpad * 256;
  const uint8_t* vx = (const uint8_t*)a.vexp + ((int64_t)b * H + h) * a.lpad * 256;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  struct Staged {
    u32x4 rk[NPK], rv[NPK], rr[NPR];
  };
  Staged set0, set1;
  auto load = [&](int kt, Staged& R) {
    const int t0 = kt * KT;
#pragma unroll
    for (int e = 0; e < NPK; ++e) {
      const int idx = tid + 256 * e, row = idx >> 4, pc = idx & 15;
      const int t = min(t0 + row, len - 1);
      R.rk[e] = *(const u32x4*)(kx + (int64_t)t * 256 + pc * 16);
      R.rv[e] = *(const u32x4*)(vx + (int64_t)t * 256 + pc * 16);
    }
    const int page = bt_row[t0 / kPage];
#pragma unroll
    for (int e = 0; e < NPR; ++e) {
      const int idx = tid + 256 * e, row = idx >> 3, pc = idx & 7;
      const int t = min(t0 + row, len - 1);
      const int pg = (t / kPage == t0 / kPage) ? page : bt_row[t / kPage];
      R.rr[e] = *(const u32x4*)((const uint8_t*)a.kv_rope +
                              ((int64_t)pg * kPage + (t % kPage)) * (D_ROPE * 2) + pc * 16);
    }
  };
  auto store = [&](int st, const Staged& R) {
    uint8_t* s = s_kv[st];
#pragma unroll
    for (int e = 0; e < NPK; ++e) {
      const int idx = tid + 256 * e, row = idx >> 4, pc = idx & 15;
      *(u32x4*)(s + K_OFF + row * K_PITCH + pc * 16) = R.rk[e];
      *(u32x4*)(s + V_OFF + row * V_PITCH + pc * 16) = R.rv[e];
    }
#pragma unroll
    for (int e = 0; e < NPR; ++e) {
      const int idx = tid + 256 * e, row = idx >> 3, pc = idx & 7;
      *(u32x4*)(s + R_OFF + row * R_PITCH + pc * 16) = R.rr[e];
    }
  };

  f32x16 o[D_V / 32];
#pragma unroll
  for (int db = 0; db < D_V / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // one key tile from stage st
  auto tile_step = [&](int kt, int st) {
    const uint8_t* s = s_kv[st];
    const int t0 = kt * KT;
    // scores of the two 32-key blocks: every K operand is read into its own
    // registers first, then the two blocks' MFMA chains alternate (a read
    // waited for right before its MFMA would cost the MFMA an LDS round trip)
    u16x8 kv[NBK][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk) {
        const int key = 32 * bk + lc;
        kv[bk][ks] = ks < KS_N
                         ? *(const u16x8*)(s + K_OFF + key * K_PITCH + (ks * 16 + hh * 8) * 2)
                         : *(const u16x8*)(s + R_OFF + key * R_PITCH +
                                           ((ks - KS_N) * 16 + hh * 8) * 2);
      }
    f32x16 sc[NBK];
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) sc[bk] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk) sc[bk] = mfma32(kv[bk][ks], q[ks], sc[bk]);
    // the V^T operands of the output product, read now so that they land
    // while the softmax runs: k-step (bk, kb) covers keys
    // 32bk + 16kb + {4hh + r, 8 + 4hh + r}
    const int g1 = (lane >> 4) & 1, r = (lane & 15) >> 2, qd = lane & 3;
    u16x8 va[NBK][2][D_V / 32];
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = 32 * bk + 16 * kb + 4 * hh + r;
#pragma unroll
        for (int db = 0; db < D_V / 32; ++db) {
          const uint8_t* p = s + V_OFF + key * V_PITCH + (32 * db + 16 * g1 + 4 * qd) * 2;
          const u16x4 lo4 = lds_read_tr16((const MLA_LDS uint8_t*)(p));
          const u16x4 hi4 = lds_read_tr16((const MLA_LDS uint8_t*)(p + 8 * V_PITCH));
          va[bk][kb][db] = u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        }
      }
    // online softmax (log2 units); lane: row lc, keys 32bk + 8(i >> 2) + 4hh + (i & 3).
    // x holds the raw scores (keys past a row's limit: -inf, applied only on
    // tiles that some row of the wave does not see whole); the scale
    // (positive) goes into the maximum here and into the exponent's FMA below
    float x[NBK][16];
    float mt = -INFINITY;
    if (__ballot(t0 + KT > lim) == 0) {
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x[bk][i] = sc[bk][i];
          mt = fmaxf(mt, x[bk][i]);
        }
    } else {
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = t0 + 32 * bk + 8 * (i >> 2) + 4 * hh + (i & 3);
          x[bk][i] = t < lim ? sc[bk][i] : -INFINITY;
          mt = fmaxf(mt, x[bk][i]);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * a.scale_log2;
    // Lazy rescaling: a row's reference m moves only when the tile's maximum
    // passes it by more than kLazy log2 units, so probabilities up to 2^kLazy
    // stay in P (fine in bf16 and in the fp32 sums) and most tiles skip the
    // output rescale; the wave takes it when any of its rows needs it.  A row
    // with no visible key yet keeps m = -inf and P = 0.
    const bool grow = mt > m + kLazy;
    if (__ballot(grow)) {
      const float mn = grow ? mt : m;
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D_V / 32; ++db) o[db] *= alpha;
      m = mn;
    }
    const float msub = m == -INFINITY ? 0.f : m;
    u16x8 pk[NBK][2];
    float psum = 0.f;
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t w4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 8 * kb + 2 * c;
          w4[c] = pack_bf16x2(fast_exp2(fmaf(x[bk][i], a.scale_log2, -msub)),
                              fast_exp2(fmaf(x[bk][i + 1], a.scale_log2, -msub)));
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w4[c]), one2, psum,
                                                 false);
        }
        pk[bk][kb] = __builtin_bit_cast(u16x8, u32x4{w4[0], w4[1], w4[2], w4[3]});
      }
    l += psum;
    // O^T += V^T P^T
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int db = 0; db < D_V / 32; ++db) o[db] = mfma32(va[bk][kb][db], pk[bk][kb], o[db]);
  };
  // Tile kt sits in stage kt & 1 and is read while the loads of tile kt + 2
  // are in flight; then tile kt + 1 (loaded during the previous tile) is
  // stored to the other stage, whose tile kt - 1 every wave left at the last
  // barrier, and the barrier publishes it.
  if (ntiles > 0) load(0, set0);
  if (ntiles > 1) load(1, set1);
  if (ntiles > 0) store(0, set0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; kt += 2) {
    if (kt + 2 < ntiles) load(kt + 2, set0);
    tile_step(kt, 0);
    if (kt + 1 >= ntiles) break;
    store(1, set1);
    __syncthreads();
    if (kt + 3 < ntiles) load(kt + 3, set1);
    tile_step(kt + 1, 1);
    if (kt + 2 >= ntiles) break;
    store(0, set0);
    __syncthreads();
  }
  // normalise and store: lane holds row lc, dims 32db + 8(i >> 2) + 4hh + (i & 3)
  const float lsum = l + __shfl_xor(l, 32, 64);
  if (!row_ok) return;
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* out = (uint16_t*)a.out + (((int64_t)b * a.q_len + j) * H + h) * D_V;
#pragma unroll
  for (int db = 0; db < D_V / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(u32x2*)(out + 32 * db + 8 * g + 4 * hh) =
          u32x2{pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
  if (a.lse != nullptr && hh == 0)
    a.lse[((int64_t)b * a.q_len + j) * H + h] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  // slices of at most EX_MAX_SLICE tiles, enough of them for about 512 workgroups
  const int max_tiles = (a.lpad + EX_T - 1) / EX_T;
  const int want = (512 + 2 * a.n_heads * a.batch - 1) / (2 * a.n_heads * a.batch);
  int slices = max((max_tiles + EX_MAX_SLICE - 1) / EX_MAX_SLICE, min(want, max_tiles));
  if (slices < 1) slices = 1;
  const int slice_tiles = (max_tiles + slices - 1) / slices;
  slices = (max_tiles + slice_tiles - 1) / slice_tiles;
  hipLaunchKernelGGL(expand_kv_kernel, dim3(2 * a.n_heads, a.batch, slices), dim3(256), 0, s, a,
                     slice_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_kernel, dim3((a.q_len + QB - 1) / QB, a.n_heads, a.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace mla
