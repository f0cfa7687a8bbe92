// Split-KV MLA decode over the paged latent cache, bf16 latent, gfx950.
//
// What it computes (one workgroup = 128 (query token, head) rows of one
// sequence and one chunk, a contiguous range of 32-token tiles, of its cache):
//   s[t]   = scale * ( q~ . c_t + q_pe . k^R_t )        (absorbed query, see
//            "Multi-Head Latent Attention: Scaling LLM Serving Throughput via
//            Low-Rank KV Compression", section "Empirical Gains", paragraph
//            on absorbing W^UK into the query side; the cache holds only c_t
//            and k^R_t per token, same section)
//   o~     = sum_t softmax(s)_t c_t                      (the latent output;
//            W^UV is applied by the combine pass)
// and the chunk's partial (o~ normalised by its own softmax sum, and its
// natural-log log-sum-exp) for the combine pass.
//
// Mapping onto CDNA4:
//   * 4 waves, wave w owns rows 32w..32w+31 (two 16-row MFMA blocks).  Its
//     absorbed query [32 x 576] bf16 stays in VGPRs (144 regs) and its output
//     accumulator [32 x 512] f32 in AGPRs (256 regs) for the whole chunk.
//   * The 32-token tile [c ; k^R] (32 x 1152 B) is brought from HBM straight
//     into LDS with 16-byte global_load_lds (no VGPR staging), through a ring
//     of 4 stages so three tiles are in flight while one is consumed.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows from LDS
//     (ds_read_b128), B = the query from registers.  The accumulator leaves
//     each lane with one head and 8 tokens, which is exactly the B operand of
//     the next product, so the probabilities never touch LDS.
//   * O^T += C^T P^T with the same MFMA: A = C^T read with ds_read_b64_tr_b16
//     (the LDS transpose read), B = P from registers.
//   * Online softmax in fp32 (base 2, scale folded).  Each row keeps a fixed
//     reference maximum instead of rescaling the accumulator every time the
//     maximum grows: probabilities are exp2(s - m_ref) <= 2^64, so nothing
//     overflows.  If a tile's maximum exceeds m_ref + 64, the accumulated part
//     is merged into the row's partial slot (log-sum-exp weights) and the
//     accumulator restarts at the new reference.  The accumulator is thus
//     only ever written by MFMAs, which keeps it resident in AGPRs.
//   * LDS rows are XOR-swizzled on 16-byte chunks (chunk c of token t is
//     stored at c ^ (t & 7)) so both read patterns spread over the banks.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int D_LAT = 512;
constexpr int D_ROPE = 64;
constexpr int LAT_ROW = D_LAT * 2;         // bytes per cached latent row
constexpr int ROPE_ROW = D_ROPE * 2;       // bytes per cached rotary row
constexpr int KS_LAT = D_LAT / 32;         // QK k-steps over the latent
constexpr int KS_ROPE = D_ROPE / 32;       // QK k-steps over the rotary part
constexpr int KS = KS_LAT + KS_ROPE;
constexpr int DB = D_LAT / 16;             // PV output column blocks
constexpr int LAT_STAGE = kTile * LAT_ROW;   // 32 KiB
constexpr int ROPE_STAGE = kTile * ROPE_ROW; // 4 KiB
constexpr int STAGE = LAT_STAGE + ROPE_STAGE;
constexpr int NSTAGE = 4;
constexpr float kRefSlack = 64.0f;         // log2 units

__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

// Issue the 9 DMA instructions of this wave for tile k of sequence b into
// stage st.  Tokens past the end of the sequence re-read its last token
// (finite data that the mask then ignores), so every wave issues the same count.
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, int b, int len, int k, int st,
                                           int w, int lane) {
  const int tok0 = k * kTile;
  const int last = len - 1;
  const int page = sload_i32(a.block_table + (int64_t)b * a.max_pages, tok0 / kPage);
  const int64_t row0 = (int64_t)page * kPage + (tok0 % kPage);
  // uniform 64-bit bases (SGPRs) + 32-bit per-lane offsets
  const uint8_t* lat = (const uint8_t*)a.kv_lat + row0 * LAT_ROW;
  const uint8_t* rope = (const uint8_t*)a.kv_rope + row0 * ROPE_ROW;
  MLA_LDS uint8_t* dst = stage_base(st);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int t = w * 8 + q;
    const int tc = min(tok0 + t, last) - tok0;
    dma16(lat + tc * LAT_ROW + (uint32_t)((lane ^ q) << 4), dst + t * LAT_ROW);
  }
  {
    const int t = w * 8 + (lane >> 3);
    const int tc = min(tok0 + t, last) - tok0;
    const uint32_t off = (uint32_t)(tc * ROPE_ROW + (((lane & 7) ^ (lane >> 3)) << 4));
    dma16(rope + off, dst + LAT_STAGE + w * 8 * ROPE_ROW);
  }
}

__device__ __forceinline__ void wait_tiles(int remaining_after) {
  // this wave's DMA for the current tile is done once at most
  // 9 * min(2, remaining_after) of its newer VMEM ops are outstanding
  if (remaining_after >= 2) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if (remaining_after == 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Eight LDS transpose reads (4 column blocks x the two 16-token halves) and a
// wait for them, in one asm block.  Written as asm because the compiler cannot
// tell that these reads never touch the stages the DMA is still filling, and
// would otherwise drain every outstanding global->LDS copy before each read.
template <int OFF>
__device__ __forceinline__ void tr_read4(const MLA_LDS uint8_t* p0, const MLA_LDS uint8_t* p1,
                                         const MLA_LDS uint8_t* p2, const MLA_LDS uint8_t* p3,
                                         u32x2 (&r)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "i"(OFF), "i"(OFF + 16 * LAT_ROW)
      : "memory");
}

struct SegState {
  u16x8 q[2][KS];       // absorbed query (B operand), per 16-row block
  f32x4 o[2][DB];       // O^T accumulator: lane holds head lr, 4 latent dims
  float m[2], l[2];     // reference max (log2 units, scaled) and per-lane sum
  int lim[2];           // keys visible to the lane's row: t < lim
  bool dumped;          // the slot already holds an earlier part of this chunk
};

// Bank the accumulated part of the chunk in its partial slot.
// The slot holds the chunk's output so far, normalised, and its natural-log
// log-sum-exp.  The first time, the slot receives O / l directly.  Later
// times (a row's scores jumped far above its reference mid-chunk) the raw
// accumulator is stored to the slot's scratch rows first and read back, so
// the merge arithmetic runs on loaded copies and the accumulator itself is
// only ever touched by MFMAs and stores.
__device__ __forceinline__ void flush_to_slot(const DecodeArgs& a, SegState& S, int64_t slot,
                                              int w, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float lsum = S.l[hb];
    lsum = wave_sum_xor(lsum, 16);
    lsum = wave_sum_xor(lsum, 32);
    const float lse_c = lsum > 0.f ? (S.m[hb] + __log2f(lsum)) * kLn2 : -INFINITY;
    const int row = w * 32 + hb * 16 + lr;
    float* dst = a.part_o + (slot * kRowsPerWG + row) * D_LAT + lg * 4;
    float* lse_dst = a.part_lse + slot * kRowsPerWG + row;
    if (!S.dumped) {
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(f32x4*)(dst + db * 16) = S.o[hb][db] * inv;
      if (lg == 0) *lse_dst = lse_c;
    } else {
      float* tmp = a.part_tmp + (slot * kRowsPerWG + row) * D_LAT + lg * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(f32x4*)(tmp + db * 16) = S.o[hb][db];
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
      const float lse_d = *lse_dst;
      const float mx = fmaxf(lse_d, lse_c);
      const float wd = (lse_d == -INFINITY) ? 0.f : __expf(lse_d - mx);
      const float wc = (lse_c == -INFINITY) ? 0.f : __expf(lse_c - mx);
      const float tot = wd + wc;
      const float fd = tot > 0.f ? wd / tot : 0.f;
      const float fc = (tot > 0.f && lsum > 0.f) ? wc / (tot * lsum) : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 prev = *(const f32x4*)(dst + db * 16);
        if (fd == 0.f) prev = f32x4{0.f, 0.f, 0.f, 0.f};   // the slot may hold garbage
        const f32x4 cur = *(const f32x4*)(tmp + db * 16);
        *(f32x4*)(dst + db * 16) = prev * fd + cur * fc;
      }
      if (lg == 0) *lse_dst = tot > 0.f ? mx + __logf(tot) : -INFINITY;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
}

__device__ __forceinline__ void compute_tile(const DecodeArgs& a, SegState& S, int64_t slot,
                                             int st, int tok0, int w, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const MLA_LDS uint8_t* lat = stage_base(st);
  const MLA_LDS uint8_t* rope = lat + LAT_STAGE;

  // ---- S^T[t, h] = K[t, :] . Q[h, :]
  f32x4 sacc[2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) sacc[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int f = lr & 7;                         // swizzle key of rows lr and 16 + lr
  const int pe = (lg ^ f) << 4;                 // chunk position for even k-steps
  const int po = ((4 + lg) ^ f) << 4;           // ... odd k-steps
  const MLA_LDS uint8_t* lat_e = lat + lr * LAT_ROW + pe;
  const MLA_LDS uint8_t* lat_o = lat + lr * LAT_ROW + po;
  const MLA_LDS uint8_t* rope_e = rope + lr * ROPE_ROW + pe;
  const MLA_LDS uint8_t* rope_o = rope + lr * ROPE_ROW + po;
  auto load_k = [&](int kk, int tb) -> u16x8 {
    if (kk < KS_LAT)
      return *(const MLA_LDS u16x8*)(((kk & 1) ? lat_o : lat_e) + tb * 16 * LAT_ROW +
                                     (kk >> 1) * 128);
    const int k2 = kk - KS_LAT;
    return *(const MLA_LDS u16x8*)(((k2 & 1) ? rope_o : rope_e) + tb * 16 * ROPE_ROW +
                                   (k2 >> 1) * 128);
  };
  u16x8 nxt0 = load_k(0, 0), nxt1 = load_k(0, 1);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const u16x8 cur0 = nxt0, cur1 = nxt1;
    if (kk + 1 < KS) {
      nxt0 = load_k(kk + 1, 0);
      nxt1 = load_k(kk + 1, 1);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sacc[0][hb] = mfma_bf16_16x16x32(cur0, S.q[hb][kk], sacc[0][hb]);
      sacc[1][hb] = mfma_bf16_16x16x32(cur1, S.q[hb][kk], sacc[1][hb]);
    }
  }

  // ---- online softmax; lane holds head (hb*16 + lr), tokens tb*16 + lg*4 + r
  float sv[2][2][4];
  float mt[2];
  bool need[2];
  bool dump = false;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + tb * 16 + lg * 4 + r;
        const float v = (t < S.lim[hb]) ? sacc[tb][hb][r] * a.scale_log2 : -INFINITY;
        sv[hb][tb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    mt[hb] = mx;
    need[hb] = mx > S.m[hb] + kRefSlack;
    dump |= need[hb] && (S.l[hb] > 0.f);
  }
  if (__ballot(dump)) {
    // rare: a row's scores jumped far above its reference; bank what has
    // been accumulated and restart from the new reference
    if (!S.dumped) {
      // an empty slot merges as log-sum-exp -inf
      if (lg == 0) {
        a.part_lse[slot * kRowsPerWG + w * 32 + lr] = -INFINITY;
        a.part_lse[slot * kRowsPerWG + w * 32 + 16 + lr] = -INFINITY;
      }
      S.dumped = true;
    }
    flush_to_slot(a, S, slot, w, lane);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int db = 0; db < DB; ++db) S.o[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      S.l[hb] = 0.f;
    }
  }
  u16x8 pf[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (need[hb]) S.m[hb] = mt[hb];
    const float mref = S.m[hb];
    uint32_t pk[4];
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = (mref == -INFINITY) ? 0.f : exp2f(sv[hb][tb][r] - mref);
        const float p1 = (mref == -INFINITY) ? 0.f : exp2f(sv[hb][tb][r + 1] - mref);
        const uint32_t u = pack_bf16x2(p0, p1);
        pk[tb * 2 + r / 2] = u;
        psum += __uint_as_float(u << 16) + __uint_as_float(u & 0xffff0000u);
      }
    S.l[hb] += psum;
    pf[hb] = __builtin_bit_cast(u16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
  }

  // ---- O^T[d, h] += C^T[d, t] P^T[t, h]
  // transpose read: lane (lg, lr) addresses token row lg*4 + lr/4 (and +16),
  // latent dims db*16 + (lr&3)*4 .. +3, i.e. chunk 2db + (lr&3)/2
  const int t1 = lg * 4 + (lr >> 2);
  const int f1 = t1 & 7;
  const int cbit = (lr & 3) >> 1;
  const int half = (lr & 1) << 3;
  const MLA_LDS uint8_t* p0 = lat + t1 * LAT_ROW + (((0 + cbit) ^ f1) << 4) + half;
  const MLA_LDS uint8_t* p1 = lat + t1 * LAT_ROW + (((2 + cbit) ^ f1) << 4) + half;
  const MLA_LDS uint8_t* p2 = lat + t1 * LAT_ROW + (((4 + cbit) ^ f1) << 4) + half;
  const MLA_LDS uint8_t* p3 = lat + t1 * LAT_ROW + (((6 + cbit) ^ f1) << 4) + half;
#pragma unroll
  for (int bat = 0; bat < DB / 4; ++bat) {
    u32x2 r[8];
    switch (bat) {
      case 0: tr_read4<0 * 128>(p0, p1, p2, p3, r); break;
      case 1: tr_read4<1 * 128>(p0, p1, p2, p3, r); break;
      case 2: tr_read4<2 * 128>(p0, p1, p2, p3, r); break;
      case 3: tr_read4<3 * 128>(p0, p1, p2, p3, r); break;
      case 4: tr_read4<4 * 128>(p0, p1, p2, p3, r); break;
      case 5: tr_read4<5 * 128>(p0, p1, p2, p3, r); break;
      case 6: tr_read4<6 * 128>(p0, p1, p2, p3, r); break;
      default: tr_read4<7 * 128>(p0, p1, p2, p3, r); break;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int db = bat * 4 + v;
      const u16x8 av = __builtin_bit_cast(u16x8, u32x4{r[2 * v][0], r[2 * v][1],
                                                       r[2 * v + 1][0], r[2 * v + 1][1]});
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) S.o[hb][db] = mfma_bf16_16x16x32(av, pf[hb], S.o[hb][db]);
    }
  }
}

__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int g = xcd_logical_id(blockIdx.x, gridDim.x);

  const int64_t nt = plan_total_tiles(a.seqlens, a.batch, a.row_groups, lane);
  if (nt == 0) return;
  Chunk ch;
  if (!plan_find_chunk(a.seqlens, a.batch, a.row_groups, nt, a.num_wg, g, lane, ch)) return;
  const int k0 = (int)((int64_t)ch.c * ch.tiles / ch.splits);
  const int k1 = (int)((int64_t)(ch.c + 1) * ch.tiles / ch.splits);
  const int n = k1 - k0;
  const int64_t slot = g;

  // query rows of this unit; the (query, head) row of lane (lg, lr) in 16-row
  // block hb is R = rg*128 + 32w + 16hb + lr
  const int rows_total = a.q_len * a.n_heads;
  const uint16_t* qlat = (const uint16_t*)a.q_lat;
  const uint16_t* qpe = (const uint16_t*)a.q_pe;
  SegState S;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int R = ch.rg * kRowsPerWG + w * 32 + hb * 16 + lr;
    const bool valid = R < rows_total;
    const int j = valid ? R / a.n_heads : 0;
    const int h = valid ? R % a.n_heads : 0;
    const int64_t qrow = ((int64_t)ch.b * a.q_len + j) * a.n_heads + h;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u16x8 v;
      if (kk < KS_LAT)
        v = *(const u16x8*)(qlat + qrow * D_LAT + kk * 32 + lg * 8);
      else
        v = *(const u16x8*)(qpe + qrow * D_ROPE + (kk - KS_LAT) * 32 + lg * 8);
      S.q[hb][kk] = valid ? v : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) S.o[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    S.m[hb] = -INFINITY;
    S.l[hb] = 0.f;
    S.lim[hb] = valid ? (a.causal ? ch.len - a.q_len + j + 1 : ch.len) : 0;
  }
  S.dumped = false;

  // prologue: three tiles in flight (issued after the query loads, so the
  // first wait below covers both)
  issue_tile(a, ch.b, ch.len, k0, 0, w, lane);
  if (n > 1) issue_tile(a, ch.b, ch.len, k0 + 1, 1, w, lane);
  if (n > 2) issue_tile(a, ch.b, ch.len, k0 + 2, 2, w, lane);

  for (int i = 0; i < n; ++i) {
    wait_tiles(n - 1 - i);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + 3 < n) issue_tile(a, ch.b, ch.len, k0 + i + 3, (i + 3) & 3, w, lane);
    compute_tile(a, S, slot, i & 3, (k0 + i) * kTile, w, lane);
  }
  flush_to_slot(a, S, slot, w, lane);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_bf16_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
