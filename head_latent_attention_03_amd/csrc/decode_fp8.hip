// Split-KV MLA decode over the paged latent cache with an OCP e4m3 latent and
// a per-token f32 scale (k^R stays bf16), gfx950.
//
// What it computes (one workgroup = 128 (query token, head) rows of one
// sequence and one chunk of 32-token tiles of its cache):
//   c_t    = s_t * c^_t                               (stored e4m3 row c^_t
//            and its scale; the cache keeps c_t and k^R_t per token, see
//            "Multi-Head Latent Attention: Scaling LLM Serving Throughput
//            via Low-Rank KV Compression", section "Empirical Gains"; the
//            FP8 storage with higher-precision scaling follows "Multi-Head
//            Latent Attention - Latent KV-Cache (DeepSeek v3)", section
//            "FP8/FP32 Mixed Precision")
//   s[t]   = scale * ( q~ . c_t + q_pe . k^R_t )
//   o~     = sum_t softmax(s)_t c_t
// with the absorbed query q~ itself stored e4m3 with a per-row scale (so
// q~ . c_t = qs * s_t * (q^ . c^_t)), and the chunk's partial (o~ normalised
// by its own softmax sum, its natural-log log-sum-exp) for the combine pass.
//
// Mapping onto CDNA4:
//   * 8 waves, two per SIMD; wave w owns rows 16w..16w+15.  Its e4m3 query
//     [16 x 512] (32 regs), bf16 q_pe [16 x 64] (8 regs) and the f32 output
//     accumulator [16 x 512] (128 regs) stay in VGPRs for the whole chunk.
//   * Tile [c^ ; k^R ; s] (32 x (512 + 128 + 4) B) goes HBM -> LDS with
//     global_load_lds_dwordx4 through a ring of 6 stages (5 tiles in flight).
//   * Latent part of S^T = K Q^T: v_mfma_scale_f32_16x16x128_f8f6f4 with unit
//     block scales (A = c^ rows from LDS, B = the e4m3 query), rotary part on
//     v_mfma_f32_16x16x32_bf16 into its own accumulator; the two meet in fp32
//     with the token and row scales.
//   * O^T += C^T P'^T on v_mfma_f32_16x16x32_fp8_fp8: A = c^ columns read with
//     the 8-bit LDS transpose read (ds_read_b64_tr_b8), B = P' in e4m3 taken
//     straight from the score accumulator layout (lane = one head, 8 tokens).
//   * P' = 2^(s - m + 8) * s_t / s_ref: e4m3 with the row maximum at 256 and
//     the token scale folded in relative to s_ref, the largest token scale of
//     the chunk; O accumulates in units of s_ref / 256.  m is a running row
//     maximum; when a tile's maximum passes m + 0.75 (P' would leave e4m3's
//     range) m moves to it and O and the sum are rescaled.  The sum l adds
//     the e4m3-rounded P' back at 1 / (256 s_t / s_ref), so numerator and
//     denominator carry the same rounding.
//   * LDS rows are XOR-swizzled on 16-byte chunks (latent chunk c of token t
//     at c ^ lat8_key(t)) so that the QK reads and the transpose reads are
//     bank-conflict free; each lane's addresses are one base XOR constants.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int D_LAT = 512;
constexpr int D_ROPE = 64;
constexpr int LAT_ROW = D_LAT;                // bytes per cached e4m3 latent row
constexpr int ROPE_ROW = D_ROPE * 2;          // bytes per cached bf16 rotary row
constexpr int KS_LAT = D_LAT / 128;           // fp8 QK k-steps (K = 128)
constexpr int KS_ROPE = D_ROPE / 32;          // bf16 QK k-steps (K = 32)
constexpr int DB = D_LAT / 16;                // PV output column blocks
constexpr int ROPE_OFF = kTile * LAT_ROW;     // 16 KiB
constexpr int SCALE_OFF = ROPE_OFF + kTile * ROPE_ROW;  // 20 KiB
constexpr int STAGE = 21 * 1024;
constexpr int NSTAGE = 6;
constexpr int AHEAD = NSTAGE - 1;             // tiles in flight
constexpr int NW = 8;                         // waves, 16 rows each
constexpr int DMA_PER_TILE = 4;               // per wave: 2 latent, 1 rotary, 1 scale
constexpr float kShift = 8.0f;                // the row maximum maps to P' = 256
constexpr float kSlack = 0.75f;               // P' <= 2^8.75 < 448 between rescales

__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];

// swizzle keys: latent chunk c (0..31) of token t sits at c ^ lat8_key(t);
// rotary chunk c (0..7) at c ^ rope_key(t)
__device__ __forceinline__ int lat8_key(int t) { return (t & 15) ^ (((t >> 4) & 1) << 3); }
__device__ __forceinline__ int rope_key(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(8))) uint32_t u32x8;

__device__ __forceinline__ u32x8 u32x8_of(u32x4 lo, u32x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// This wave's 4 DMA instructions for tile k, whose first token sits in
// physical page `page`: latent rows of tokens 4w..4w+3 (two 1 KiB copies),
// their rotary rows (32 lanes) and their 4 scales (one lane).  Latent and
// rotary rows past the sequence end re-read its last token; the scales of
// such tokens are whatever the page holds and are never used unmasked.
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, int page, int len, int k, int st,
                                           int w, int lane) {
  const int tok0 = k * kTile;
  const int last = len - 1;
  const int64_t row0 = (int64_t)page * kPage + (tok0 % kPage);
  const uint8_t* lat = (const uint8_t*)a.kv_lat + row0 * LAT_ROW;
  const uint8_t* rope = (const uint8_t*)a.kv_rope + row0 * ROPE_ROW;
  MLA_LDS uint8_t* dst = stage_base(st);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // lane l fills row 4w + 2j + l/32 at chunk position l % 32
    const int t = w * 4 + 2 * j + (lane >> 5);
    const int tc = min(tok0 + t, last) - tok0;
    const uint32_t off = (uint32_t)(tc * LAT_ROW + (((lane & 31) ^ lat8_key(t)) << 4));
    dma16_s(lat, off, dst + (w * 4 + 2 * j) * LAT_ROW);
  }
  {
    const int t = w * 4 + (lane >> 3);
    const int tc = min(tok0 + t, last) - tok0;
    const uint32_t off = (uint32_t)(tc * ROPE_ROW + (((lane & 7) ^ rope_key(t)) << 4));
    if (lane < 32) dma16_s(rope, off, dst + ROPE_OFF + w * 4 * ROPE_ROW);
  }
  if (lane == 0) dma16_s(a.kv_scale + row0 + w * 4, 0u, dst + SCALE_OFF + w * 16);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The current tile's copies are done once at most
// DMA_PER_TILE * min(AHEAD - 1, remaining_after) newer ones are outstanding.
__device__ __forceinline__ void wait_tiles(int remaining_after) {
  switch (remaining_after < AHEAD - 1 ? remaining_after : AHEAD - 1) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<DMA_PER_TILE>(); break;
    case 2: wait_vm<2 * DMA_PER_TILE>(); break;
    case 3: wait_vm<3 * DMA_PER_TILE>(); break;
    default: wait_vm<4 * DMA_PER_TILE>(); break;
  }
}
static_assert(AHEAD - 1 == 4, "wait_tiles covers up to 4 newer tiles");

struct State {
  i32x8 q8[KS_LAT];     // e4m3 query, 32 bytes per k-step (B operand)
  u16x8 qpe[KS_ROPE];   // bf16 rotary query (B operand)
  f32x4 o[DB];          // O^T accumulator: lane holds head lr, 4 latent dims
  float qs;             // the row's query scale
  float m, l;           // running max (log2 units, scaled) and per-lane sum
  int lim;              // keys visible to the lane's row: t < lim
};

// Per-lane LDS byte offsets from a stage's base.  Every address a tile reads
// is one of them XOR a constant:
//   QK latent, k-step kk, half h, block tb:  qk ^ (kk << 7) ^ (h << 4) ^ tb * (8192 | 128)
//   QK rotary, k-step v, block tb:           rp ^ (v << 6), + tb * 16 rows
//   PV transpose, column block db:           pv ^ (db << 4)
struct LaneOff {
  uint32_t qk, rp, pv;
};

__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  LaneOff o;
  o.qk = (uint32_t)(lr * LAT_ROW + (((2 * lg) ^ lat8_key(lr)) << 4));
  o.rp = (uint32_t)(ROPE_OFF + lr * ROPE_ROW + ((lg ^ rope_key(lr)) << 4));
  // transpose read: in lane group lg, lane n addresses row n/2 of the 8-row
  // block, bytes 8(n&1)..+7; row r is token lg*4 + r (r < 4) or
  // 16 + lg*4 + r - 4, the tokens this lane group holds P' for
  const int r = lr >> 1;
  const int tok = (r < 4) ? lg * 4 + r : 16 + lg * 4 + (r - 4);
  o.pv = (uint32_t)(tok * LAT_ROW + (lat8_key(tok) << 4) + ((lr & 1) << 3));
  return o;
}

__device__ __forceinline__ f32x4 mfma_fp8_k128(i32x8 a, i32x8 b, f32x4 c) {
  // e4m3 x e4m3, unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ f32x4 mfma_fp8_k32(long a, long b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void compute_tile(const DecodeArgs& a, State& S, int st, int tok0,
                                             int lane, LaneOff lo, float inv_sref,
                                             float sref_256) {
  const int lg = lane >> 4;
  const MLA_LDS uint8_t* base = stage_base(st);
  asm volatile("" : "+v"(lo.qk), "+v"(lo.rp), "+v"(lo.pv));

  // ---- latent scores (fp8) and rotary scores (bf16), S^T[t, h]
  f32x4 sl[2], sr[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    sl[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    sr[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto load_k8 = [&](int kk, int tb) -> i32x8 {
    const uint32_t o0 = lo.qk ^ (uint32_t)(kk << 7) ^ (uint32_t)(tb * (8192 | 128));
    const u32x4 x0 = *(const MLA_LDS u32x4*)(base + o0);
    const u32x4 x1 = *(const MLA_LDS u32x4*)(base + (o0 ^ 16u));
    return __builtin_bit_cast(i32x8, u32x8_of(x0, x1));
  };
  i32x8 ka[2][2];
  ka[0][0] = load_k8(0, 0);
  ka[0][1] = load_k8(0, 1);
#pragma unroll
  for (int kk = 0; kk < KS_LAT; ++kk) {
    if (kk + 1 < KS_LAT) {
      ka[(kk + 1) & 1][0] = load_k8(kk + 1, 0);
      ka[(kk + 1) & 1][1] = load_k8(kk + 1, 1);
    }
    sl[0] = mfma_fp8_k128(ka[kk & 1][0], S.q8[kk], sl[0]);
    sl[1] = mfma_fp8_k128(ka[kk & 1][1], S.q8[kk], sl[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int v = 0; v < KS_ROPE; ++v) {
    const MLA_LDS uint8_t* p = base + (lo.rp ^ (uint32_t)(v << 6));
    const u16x8 k0 = *(const MLA_LDS u16x8*)p;
    const u16x8 k1 = *(const MLA_LDS u16x8*)(p + 16 * ROPE_ROW);
    sr[0] = mfma_bf16_16x16x32(k0, S.qpe[v], sr[0]);
    sr[1] = mfma_bf16_16x16x32(k1, S.qpe[v], sr[1]);
  }

  // ---- scores; lane holds head lr and tokens tb*16 + lg*4 + r
  f32x4 sc[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
    sc[tb] = *(const MLA_LDS f32x4*)(base + SCALE_OFF + (tb * 16 + lg * 4) * 4);
  float sv[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + tb * 16 + lg * 4 + r;
      const float v = (t < S.lim)
                          ? (sl[tb][r] * (sc[tb][r] * S.qs) + sr[tb][r]) * a.scale_log2
                          : -INFINITY;
      sv[tb][r] = v;
      mx = fmaxf(mx, v);
    }
  mx = wave_max_xor(mx, 16);
  mx = wave_max_xor(mx, 32);
  // lazy rescale: move the reference only when P' would leave e4m3's range
  const bool need = mx > S.m + kSlack;
  if (__ballot(need)) {
    const float m_new = need ? mx : S.m;
    const float alpha = need ? fast_exp2(S.m - m_new) : 1.0f;  // 0 on a row's first keys
    S.m = m_new;
    S.l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) S.o[db] *= alpha;
  }

  // ---- P' = 2^(s - m + 8) * s_t / s_ref in e4m3, and l += P' * s_ref / (256 s_t)
  uint32_t pk[2];
  float lsum = 0.f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    float x[4], inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = sv[tb][r] != -INFINITY;
      x[r] = valid ? fast_exp2(sv[tb][r] - S.m + kShift) * (sc[tb][r] * inv_sref) : 0.f;
      inv[r] = valid ? sref_256 * __builtin_amdgcn_rcpf(sc[tb][r]) : 0.f;
    }
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], p, true);
    pk[tb] = (uint32_t)p;
    const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(p, false);
    const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(p, true);
    lsum += b01[0] * inv[0] + b01[1] * inv[1] + b23[0] * inv[2] + b23[1] * inv[3];
  }
  S.l += lsum;
  const long pf = (long)(((uint64_t)pk[1] << 32) | pk[0]);

  // ---- O^T[d, h] += C^T[d, t] P'^T[t, h]
  auto load_c = [&](int db) -> long {
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (MLA_LDS i32x2*)(base + (lo.pv ^ (uint32_t)(db << 4))));
    return __builtin_bit_cast(long, v);
  };
  constexpr int PV_AHEAD = 4;
  long ca[PV_AHEAD];
#pragma unroll
  for (int j = 0; j < PV_AHEAD; ++j) ca[j] = load_c(j);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const long av = ca[db % PV_AHEAD];
    if (db + PV_AHEAD < DB) ca[db % PV_AHEAD] = load_c(db + PV_AHEAD);
    S.o[db] = mfma_fp8_k32(av, pf, S.o[db]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ __launch_bounds__(64 * NW, 1) void decode_fp8_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;

  int g;
  Chunk ch;
  if (!plan_locate(a.seqlens, a.batch, a.row_groups, a.num_wg, blockIdx.x, lane, g, ch)) return;
  if (ch.c == 0 && threadIdx.x == 0) {
    const int64_t u = (int64_t)ch.b * a.row_groups + ch.rg;
    a.unit_chunks[2 * u] = g;
    a.unit_chunks[2 * u + 1] = ch.splits;
  }
  const int k0 = (int)((int64_t)ch.c * ch.tiles / ch.splits);
  const int k1 = (int)((int64_t)(ch.c + 1) * ch.tiles / ch.splits);
  const int n = k1 - k0;
  const int64_t slot = g;

  // query rows: row R = rg*128 + 16w + lr
  const int rows_total = a.q_len * a.n_heads;
  const int R = ch.rg * kRowsPerWG + w * 16 + lr;
  const bool valid = R < rows_total;
  const int j = valid ? R / a.n_heads : 0;
  const int h = valid ? R % a.n_heads : 0;
  const int64_t qrow = ((int64_t)ch.b * a.q_len + j) * a.n_heads + h;
  State S;
  {
    const uint8_t* q8 = (const uint8_t*)a.q_lat + qrow * D_LAT;
    const uint16_t* qpe = (const uint16_t*)a.q_pe + qrow * D_ROPE;
#pragma unroll
    for (int kk = 0; kk < KS_LAT; ++kk) {
      const i32x8 v = *(const i32x8*)(q8 + kk * 128 + lg * 32);
      S.q8[kk] = valid ? v : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int kk = 0; kk < KS_ROPE; ++kk) {
      const u16x8 v = *(const u16x8*)(qpe + kk * 32 + lg * 8);
      S.qpe[kk] = valid ? v : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    S.qs = valid ? a.q_scale[qrow] : 0.f;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) S.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  S.m = -INFINITY;
  S.l = 0.f;
  S.lim = valid ? (a.causal ? ch.len - a.q_len + j + 1 : ch.len) : 0;

  // page indices of the chunk, one per lane (a window of 64)
  const int32_t* bt_row = a.block_table + (int64_t)ch.b * a.max_pages;
  PageWindow W;
  W.pg0 = uni(k0 * kTile / kPage);
  W.v = page_window_load(bt_row, a.max_pages, W.pg0, lane);
  auto issue = [&](int k, int st) {
    issue_tile(a, page_lookup(W, bt_row, a.max_pages, k * kTile / kPage, lane), ch.len, k, st, w,
               lane);
  };

  // prologue: AHEAD tiles in flight
#pragma unroll
  for (int i = 0; i < AHEAD; ++i)
    if (i < n) issue(k0 + i, i);

  // s_ref: the largest token scale of the chunk (every wave forms it alone)
  float sref = 0.f;
  {
    const int t_end = min(k1 * kTile, ch.len);
    const int32_t* bt = a.block_table + (int64_t)ch.b * a.max_pages;
    for (int t = k0 * kTile + lane; t < t_end; t += 64) {
      const int page = bt[t / kPage];
      sref = fmaxf(sref, a.kv_scale[(int64_t)page * kPage + (t % kPage)]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sref = fmaxf(sref, __shfl_xor(sref, m, 64));
    if (!(sref > 0.f)) sref = 1.f;
  }
  const float inv_sref = 1.0f / sref;
  const float sref_256 = sref * (1.0f / 256.0f);

  const LaneOff lo = lane_offsets(lane);
  for (int i = 0; i < n; ++i) {
    wait_tiles(n - 1 - i);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + AHEAD < n) issue(k0 + i + AHEAD, (i + AHEAD) % NSTAGE);
    compute_tile(a, S, i % NSTAGE, (k0 + i) * kTile, lane, lo, inv_sref, sref_256);
  }

  // the chunk's partial: o~ / l (bf16) and its natural-log LSE
  float lsum = S.l;
  lsum = wave_sum_xor(lsum, 16);
  lsum = wave_sum_xor(lsum, 32);
  const float lse = lsum > 0.f ? (S.m + __log2f(lsum)) * kLn2 : -INFINITY;
  const float f = lsum > 0.f ? sref_256 / lsum : 0.f;
  const int row = w * 16 + lr;
  uint16_t* dst = (uint16_t*)a.part_o + (slot * kRowsPerWG + row) * D_LAT + lg * 4;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const f32x4 v = S.o[db] * f;
    *(u32x2*)(dst + db * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
  if (lg == 0) a.part_lse[slot * kRowsPerWG + row] = lse;
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
