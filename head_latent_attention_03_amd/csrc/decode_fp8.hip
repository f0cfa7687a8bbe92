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
// Mapping onto CDNA4 (4 waves, one per SIMD, 512 registers each; the same
// plan as the bf16 kernel):
//   * Wave w owns rows 32w .. 32w+31: its e4m3 query [32 x 512] (64 VGPRs),
//     bf16 q_pe [32 x 64] (16 VGPRs) and its output accumulator [32 x 512]
//     f32 (the 256 accumulation registers).
//   * Latent scores: v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales
//     (e4m3 x e4m3; twice the bf16 rate), A = 32 c^ rows x 64 bytes from LDS
//     (two ds_read_b128 per lane), B = the query.  Rotary scores on
//     v_mfma_f32_32x32x16_bf16 into their own accumulator; the two meet in
//     fp32 with the token and row scales.  Each lane ends with head l & 31
//     and tokens 8(i >> 2) + 4(l >> 5) + (i & 3).
//   * O^T += C^T P'^T on v_mfma_f32_32x32x16_fp8_fp8: A = c^ columns, one
//     ds_read_b64_tr_b8 (the 8-bit LDS transpose read) per lane and MFMA,
//     rows taken in the order the score accumulator holds the tokens; B = P'
//     in e4m3 straight from the score registers.
//   * P' = 2^(s - m + 8) * s_t / s_ref: e4m3 with the row maximum at 256 and
//     the token scale folded in relative to s_ref, the largest token scale of
//     the chunk; O accumulates in units of s_ref / 256.  m is a fixed row
//     reference set by the row's first visible scores and never moved, so O
//     is never rescaled.  A later score past m + 0.75 (where P' would leave
//     e4m3's range) sends the whole workgroup through a second pass with the
//     row's true maximum as m.  The sum l adds the e4m3-rounded P' back at
//     s_ref / (256 s_t), so numerator and denominator carry the same
//     rounding.
//   * Iteration i copies tile i + 5 and runs the output product of tile
//     i - 1 beside the scores of tile i (independent accumulators), then the
//     softmax of tile i.  A ring of 7 stages [c^ ; k^R ; s] (20.1 KiB each)
//     keeps five tiles in flight; each wave copies two latent rows per
//     instruction (4), eight rotary rows (1) and eight scales (1) per tile.
//   * LDS rows are XOR-swizzled on 16-byte chunks for gfx950's LDS (64 banks
//     of 4 bytes; a 16-byte read serves its lanes in four 16-lane cycles,
//     lanes taken in quads, the cycle of lane l being (l >> 5, parity of
//     bits 2..4 of l); an 8-byte transpose read serves lanes 0-31, then
//     32-63).  Latent chunk c of token t sits at slot (c & 15) ^ key(t) of its
//     256-byte group, key(t) = 4(t & 3) + ((t >> 2) & 3):
//       - scores: a cycle's 16 lanes read one chunk of 16 tokens 4a + r
//         whose a share a parity; (r, a & 3) takes each of its 16 values once;
//       - transpose: a half-wave reads 2 adjacent chunks of 8 tokens
//         16kb + 4hh + r and 16kb + 8 + 4hh + r (r < 4), whose keys
//         4r + hh and 4r + hh + 2 fill the 16 slots with the chunk bit.
//     Rotary chunk c (0..7) of token t sits at c ^ rope_key(t), rope_key(t)
//     = ((t >> 2) & 3) + 4((t >> 1) & 1), as in the bf16 kernel.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int D_LAT = 512;
constexpr int D_ROPE = 64;
constexpr int LAT_ROW = D_LAT;                // bytes per cached e4m3 latent row
constexpr int ROPE_ROW = D_ROPE * 2;          // bytes per cached bf16 rotary row
constexpr int KS_LAT = D_LAT / 64;            // fp8 score k-steps (K = 64)
constexpr int KS_ROPE = D_ROPE / 16;          // bf16 score k-steps (K = 16)
constexpr int KS = KS_LAT + KS_ROPE;          // 12
constexpr int DB = D_LAT / 32;                // 32-dim output blocks
constexpr int PV_STEPS = 2 * DB;              // two 16-token k-steps per tile
constexpr int ROPE_OFF = kTile * LAT_ROW;     // 16 KiB
constexpr int SCALE_OFF = ROPE_OFF + kTile * ROPE_ROW;  // 20 KiB
constexpr int STAGE = 21 * 1024;
constexpr int NSTAGE = 7;
constexpr int AHEAD = NSTAGE - 2;             // tiles in flight (5)
constexpr int NW = kRowsPerWG / 32;           // 4 waves
constexpr int kThreads = 64 * NW;
constexpr int kDma = 6;                       // copies per wave and tile
constexpr float kShift = 8.0f;                // the row maximum maps to P' = 256
constexpr float kSlack = 0.75f;               // P' <= 2^8.75 < 448 between rescales

__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];
__shared__ int s_flag[NW];
// per wave and tile, the per-token factors of the softmax: s_t / s_ref and
// s_ref / (256 s_t) (0 past the sequence end)
__shared__ __attribute__((aligned(16))) float s_tok[NW][2][kTile];
static_assert(SCALE_OFF + kTile * 4 <= STAGE, "stage layout");

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) uint32_t u32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;

__device__ __forceinline__ int lat_key(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int rope_key(int t) { return ((t >> 2) & 3) | (((t >> 1) & 1) << 2); }

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

__device__ __forceinline__ f32x16 mfma_lat(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3, unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ f32x16 mfma_rope(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// acc += A B (e4m3 x e4m3) with the accumulator pinned to the accumulation
// registers, which hold exactly the wave's output; each block is updated by
// MFMAs only, at least 15 MFMAs apart, and mfma_drain() covers the MFMA
// latency before anything else reads or writes the accumulators.
__device__ __forceinline__ void mfma_pv(f32x16& acc, long a, long b) {
  asm("v_mfma_f32_32x32x16_fp8_fp8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// The copies of one tile: wave w's latent rows 8w .. 8w+7 (parts 0..3, two
// 512-byte rows each), their rotary rows (part 4) and their scales (part 5,
// two lanes).  Latent and rotary rows past the sequence end re-read its last
// token; the scales of such tokens are whatever the page holds and are never
// used unmasked.
struct TileCopy {
  const uint8_t* lat;
  const uint8_t* rope;
  const float* scale;
  int tok0, last, st;
};

__device__ __forceinline__ TileCopy tile_copy(const DecodeArgs& a, int page, int len, int k,
                                              int st) {
  TileCopy c;
  c.tok0 = k * kTile;
  c.last = len - 1;
  const int64_t row0 = (int64_t)page * kPage + (c.tok0 % kPage);
  c.lat = (const uint8_t*)a.kv_lat + row0 * LAT_ROW;
  c.rope = (const uint8_t*)a.kv_rope + row0 * ROPE_ROW;
  c.scale = a.kv_scale + row0;
  c.st = st;
  return c;
}

__device__ __forceinline__ void issue_part(const TileCopy& c, int j, int w, int lane) {
  MLA_LDS uint8_t* dst = stage_base(c.st);
  if (j < 4) {
    // lane l fills row 8w + 2j + (l >> 5), slot l & 15 of group (l >> 4) & 1,
    // which holds chunk ((l >> 4) & 1) * 16 + ((l & 15) ^ key)
    const int t = w * 8 + 2 * j + (lane >> 5);
    const int tc = min(c.tok0 + t, c.last) - c.tok0;
    const uint32_t off = (uint32_t)(tc * LAT_ROW + (((lane & 31) ^ lat_key(t)) << 4));
    dma16_s(c.lat, off, dst + (w * 8 + 2 * j) * LAT_ROW);
  } else if (j == 4) {
    const int t = w * 8 + (lane >> 3);
    const int tc = min(c.tok0 + t, c.last) - c.tok0;
    const uint32_t off = (uint32_t)(tc * ROPE_ROW + (((lane & 7) ^ rope_key(t)) << 4));
    dma16_s(c.rope, off, dst + ROPE_OFF + w * 8 * ROPE_ROW);
  } else {
    if (lane < 2) dma16_s(c.scale + w * 8, (uint32_t)(lane << 4), dst + SCALE_OFF + w * 32);
  }
}

__device__ __forceinline__ void issue_tile(const TileCopy& c, int w, int lane) {
#pragma unroll
  for (int j = 0; j < kDma; ++j) issue_part(c, j, w, lane);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct State {
  i32x8 q8[KS_LAT];     // e4m3 query, 32 bytes per k-step (B operand)
  u16x8 qpe[KS_ROPE];   // bf16 rotary query (B operand)
  f32x16 o[DB];         // O^T accumulator: lane holds head l & 31, 16 of the
                        // block's 32 latent dims
  float qs;             // the row's query scale times the softmax scale (log2)
                        // times s_ref
  int len;              // the sequence length
  float m, l;           // reference max (log2 units, scaled) and per-lane sum
  int lim;              // keys visible to the lane's row: t < lim
  float tmax;           // largest score this lane has seen (log2 units, scaled)
  bool redo;            // a score passed m + kSlack
};

// Per-lane LDS byte offsets from a stage's base:
//   latent scores, k-step ks, half e:  (qk ^ (((4ks & 15) ^ e) << 4)) + 256 (ks >> 2)
//   rotary scores, k-step k:           rp ^ (2k << 4)
//   transpose, block db, k-step kb:    (pv ^ ((2 (db & 7)) << 4)) + 256 (db >> 3) + 8192 kb
// (the XORed bits never carry).
struct LaneOff {
  uint32_t qk, rp, pv;
};

__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int lc = lane & 31, hh = lane >> 5;
  const int dh = (lane >> 4) & 1, n = lane & 15;
  LaneOff o;
  // scores: lane reads token lc, chunks 4ks + 2hh + e
  o.qk = (uint32_t)(lc * LAT_ROW + (((2 * hh) ^ lat_key(lc)) << 4));
  o.rp = (uint32_t)(ROPE_OFF + lc * ROPE_ROW + ((hh ^ rope_key(lc)) << 4));
  // transpose: lane n of its 16-lane group addresses row r = n >> 1 of the
  // read, token 4hh + r (r < 4) or 8 + 4hh + r - 4, bytes 8 (n & 1) of chunk
  // 2db + dh
  const int r = n >> 1;
  const int tok = (r < 4) ? 4 * hh + r : 8 + 4 * hh + (r - 4);
  o.pv = (uint32_t)(tok * LAT_ROW + ((dh ^ lat_key(tok)) << 4) + 8 * (n & 1));
  return o;
}

// The reads take the lane's absolute LDS address for a stage (stage base +
// lane offset): stage bases are multiples of 1 KiB, so the XORed bits 4..7
// commute with the add, which then happens once per stage and tile instead of
// once per read.
__device__ __forceinline__ const MLA_LDS uint8_t* lds_at(uint32_t a) {
  return (const MLA_LDS uint8_t*)(uintptr_t)a;
}

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS uint8_t* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ i32x8 load_k(uint32_t bq, int ks) {
  const uint32_t c = (uint32_t)(((4 * ks) & 15) << 4);
  const u32x4 x0 = *(const MLA_LDS u32x4*)(lds_at(bq ^ c) + (ks >> 2) * 256);
  const u32x4 x1 = *(const MLA_LDS u32x4*)(lds_at(bq ^ (c ^ 16u)) + (ks >> 2) * 256);
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ u16x8 load_r(uint32_t br, int k) {
  return *(const MLA_LDS u16x8*)lds_at(br ^ (uint32_t)((2 * k) << 4));
}

// output step j: k-step kb = j >> 4 (tokens 16kb ..), block db = j & 15
__device__ __forceinline__ long load_v(uint32_t bv, int j) {
  const int kb = j >> 4, db = j & 15;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (MLA_LDS i32x2*)(lds_at(bv ^ (uint32_t)((2 * (db & 7)) << 4)) + (db >> 3) * 256 +
                       kb * 16 * LAT_ROW));
  return __builtin_bit_cast(long, v);
}

constexpr int AH = 2;   // LDS reads run this many steps ahead of their MFMAs

// One pipeline step group: the scores of tile stage st_qk (if QK: 8 latent
// and 4 rotary MFMAs) and the output product of stage st_pv with the e4m3
// probabilities p (if PV: 32 MFMAs), issued alternately while both run, plus
// the copies of a later tile (cp), issued at the start of steps 0, 2, .. 10.
template <bool QK, bool PV, bool COPY>
__device__ __forceinline__ void tile_step(State& S, int st_qk, int st_pv, long p0, long p1,
                                          int lane, LaneOff lo, const TileCopy& cp, int w,
                                          float sr0, f32x16& sl, f32x16& sr) {
  constexpr int NSTEP = PV ? PV_STEPS : KS;
  static_assert(2 * (kDma - 1) < KS, "the copies fit in the score steps");
  const uint32_t bq = lds_addr(stage_base(st_qk)) + lo.qk;
  const uint32_t br = lds_addr(stage_base(st_qk)) + lo.rp;
  const uint32_t bv = lds_addr(stage_base(st_pv)) + lo.pv;
  i32x8 ka[AH];
  u16x8 ra[AH];
  long va[AH];
  if (QK) {
    sl = f32x16{};
    sr = f32x16{} + sr0;
  }
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    if (QK) ka[j] = load_k(bq, j);
    if (PV) va[j] = load_v(bv, j);
  }
#pragma unroll
  for (int j = 0; j < NSTEP; ++j) {
    // a copy is issued while the previous step's MFMA still runs
    if (COPY && j % 2 == 0 && j / 2 < kDma) issue_part(cp, j / 2, w, lane);
    if (QK && j < KS_LAT) {
      const i32x8 cur = ka[j % AH];
      if (j + AH < KS_LAT) ka[j % AH] = load_k(bq, j + AH);
      else ra[(j + AH - KS_LAT) % AH] = load_r(br, j + AH - KS_LAT);
      sl = mfma_lat(cur, S.q8[j], sl);
    } else if (QK && j < KS) {
      const int k = j - KS_LAT;
      const u16x8 cur = ra[k % AH];
      if (k + AH < KS_ROPE) ra[k % AH] = load_r(br, k + AH);
      sr = mfma_rope(cur, S.qpe[k], sr);
    }
    if (PV) {
      const long cur = va[j % AH];
      if (j + AH < PV_STEPS) va[j % AH] = load_v(bv, j + AH);
      mfma_pv(S.o[j & (DB - 1)], cur, (j >> 4) ? p1 : p0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The softmax of one tile.  Lane holds head l & 31 and tokens
// 8(i >> 2) + 4hh + (i & 3).  On the chunk's first tile (first) a row's
// first scores set its reference m (the row's two lanes exchange their
// maxima); later tiles use it as it is, so the output is never rescaled, and
// their rotary accumulator starts at shift = 8 - m, so that the scores arrive
// already in the exponent of P'.  A score above m + kSlack (where P' would
// leave e4m3's range) marks the workgroup for a second pass with the true row
// maxima.  Returns the e4m3 probabilities as the two B operands (tokens
// 16kb .. of k-step kb) and adds them to the lane's sum.
__device__ __forceinline__ void tile_probs(const DecodeArgs& a, State& S, const f32x16& sl,
                                           const f32x16& sr, const MLA_LDS uint8_t* base,
                                           int tok0, int w, int lane, float inv_sref,
                                           float sref_256, bool first, float shift0, long& p0,
                                           long& p1) {
  const int hh = lane >> 5;
  // the per-token factors, once per tile and wave: lane l < 32 forms token
  // l's, the lanes read back the 16 they need (LDS is in order per wave).
  // (Scales of visible tokens are normal positive numbers, a precondition of
  // the call; a zero one would make fb infinite.)
  {
    const int t = lane & 31;
    const float st = *(const MLA_LDS float*)(base + SCALE_OFF + 4 * t);
    const bool in = tok0 + t < S.len;
    const float fa = in ? st * inv_sref : 0.f;
    const float fb = in ? sref_256 * __builtin_amdgcn_rcpf(st) : 0.f;
    if (lane < 32) {
      s_tok[w][0][t] = fa;
      s_tok[w][1][t] = fb;
    }
  }
  // the factors of the lane's tokens: 4 groups of 4 consecutive tokens
  f32x4 fa[4], fb[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    fa[g] = *(const MLA_LDS f32x4*)&s_tok[w][0][8 * g + 4 * hh];
    fb[g] = *(const MLA_LDS f32x4*)&s_tok[w][1][8 * g + 4 * hh];
  }
  // scores in log2 units: the latent part is sl * s_t * qs = sl * fa * (qs
  // s_ref), and the rotary query and qs carry the softmax scale
  float sv[16];
  float mx = -INFINITY;
  const bool cut = __ballot(tok0 + kTile > S.lim) != 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = fmaf(sl[i], fa[i >> 2][i & 3] * S.qs, sr[i]);
    if (cut && tok0 + 8 * (i >> 2) + 4 * hh + (i & 3) >= S.lim) v = -INFINITY;
    sv[i] = v;
    mx = fmaxf(mx, v);
  }
  float shift;
  if (first) {
    S.tmax = fmaxf(S.tmax, mx);
    if (__ballot(mx > S.m + kSlack)) {
      const float rmx = wave_max_xor(mx, 32);
      const float mass = wave_sum_xor(S.l, 32);
      if (rmx > S.m + kSlack && mass == 0.f) S.m = rmx;
    }
    S.redo |= mx > S.m + kSlack;
    // (a row without reference has no visible key: P' = 0)
    shift = kShift - (S.m == -INFINITY ? INFINITY : S.m);
  } else {
    // the scores carry shift0 already; (-inf - -inf = NaN for a row without
    // reference, which fmaxf ignores)
    S.tmax = fmaxf(S.tmax, mx - shift0);
    S.redo |= mx > kShift + kSlack;
    shift = 0.f;
  }
  // P' = 2^(s - m + 8) * s_t / s_ref in e4m3, and l += P' * s_ref / (256 s_t)
  uint32_t pk[4];
  float lsum = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = fast_exp2(sv[4 * g + r] + shift) * fa[g][r];
    // (saturating: a probability past 448 only occurs in a pass that is redone)
    int pw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    pw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pw, true);
    pk[g] = (uint32_t)pw;
    const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(pw, false);
    const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(pw, true);
    lsum = fmaf(b01[0], fb[g][0], lsum);
    lsum = fmaf(b01[1], fb[g][1], lsum);
    lsum = fmaf(b23[0], fb[g][2], lsum);
    lsum = fmaf(b23[1], fb[g][3], lsum);
  }
  S.l += lsum;
  p0 = (long)(((uint64_t)pk[1] << 32) | pk[0]);
  p1 = (long)(((uint64_t)pk[3] << 32) | pk[2]);
}

// The chunk's one pass over its tiles [k0, k0 + n).
//   * Prologue: the page window; the loads of the chunk's token scales (for
//     s_ref, the largest of them); the copies of tiles 0 and 1; the query.
//     All of these land before the first barrier, and the query registers
//     are marked used there, so that no wait the compiler places for its
//     own loads can fall behind a later copy.  Tiles 2 .. AHEAD follow.
//   * Iteration i (1 <= i < n) waits for tile i (this wave's copies are done
//     once at most AHEAD - 1 newer tiles' are outstanding; after the barrier
//     every wave's are, and every wave is done with stage (i - 2) % NSTAGE),
//     copies tile i + AHEAD into that stage, runs the output product of tile
//     i - 1 beside the scores of tile i and then the softmax of tile i.
//     Every iteration copies one tile (past the chunk's last tile, a re-read
//     of it into a stage that is not read again), so each wait count is a
//     constant.
template <bool FIRST, typename LoadQuery>
__device__ __forceinline__ void run_pass(const DecodeArgs& a, State& S, const Chunk& ch, int k0,
                                         int n, int w, int lane, LoadQuery load_query,
                                         float& inv_sref, float& sref_256) {
  static_assert(AHEAD + 2 <= NSTAGE, "ring");
  const LaneOff lo = lane_offsets(lane);
  const int32_t* bt_row = a.block_table + (int64_t)ch.b * a.max_pages;
  PageWindow W;
  W.pg0 = uni(k0 * kTile / kPage);
  W.v = page_window_load(bt_row, a.max_pages, W.pg0, lane);
  const int k_last = k0 + n - 1;
  auto copy_of = [&](int k, int st) {
    k = min(k, k_last);
    const int page = page_lookup(W, bt_row, a.max_pages, k * kTile / kPage, lane);
    return tile_copy(a, page, ch.len, k, st);
  };
  // the chunk's token scales, pages from the window: the first 1024 tokens
  // in one batch of loads (their pages always lie in the window), the rest
  // four loads per lane and round (a direct table read past the window)
  const int t_begin = k0 * kTile, t_end = min((k_last + 1) * kTile, ch.len);
  float sref = 0.f;
  for (int t0 = t_begin + 16 * 64; FIRST && t0 < t_end; t0 += 4 * 64) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 64 * u + lane;
      const int rel = (t >> 6) - W.pg0;
      // (every lane takes part in the shuffle: a lane outside the window
      // reads the table directly)
      const int wpage = __shfl(W.v, rel & 63, 64);
      const int page = rel < 64 ? wpage : bt_row[min(t, t_end - 1) >> 6];
      v[u] = t < t_end ? a.kv_scale[(int64_t)page * kPage + (t & (kPage - 1))] : 0.f;
    }
    sref = fmaxf(sref, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  float v[16];
  if (FIRST) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = t_begin + 64 * u + lane;
      const int page = __shfl(W.v, ((t >> 6) - W.pg0) & 63, 64);
      v[u] = t < t_end ? a.kv_scale[(int64_t)page * kPage + (t & (kPage - 1))] : 0.f;
    }
  }
  issue_tile(copy_of(k0, 0), w, lane);
  issue_tile(copy_of(k0 + 1, 1), w, lane);
  if (FIRST) load_query();
  wait_vm<0>();
  if (FIRST) {
#pragma unroll
    for (int u = 0; u < 16; ++u) sref = fmaxf(sref, v[u]);
  }
  if (FIRST) {
#pragma unroll
    for (int kk = 0; kk < KS_LAT; ++kk) asm volatile("" ::"v"(S.q8[kk]));
#pragma unroll
    for (int kk = 0; kk < KS_ROPE; ++kk) asm volatile("" ::"v"(S.qpe[kk]));
    asm volatile("" ::"v"(S.qs));
    // the softmax scale (log2 units) goes into the rotary query (rounded to
    // bf16 again: 2^-9 relative on the rotary part of a score) and into the
    // row scale
#pragma unroll
    for (int kk = 0; kk < KS_ROPE; ++kk) {
      u16x8 v = S.qpe[kk];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t pr = pack_bf16x2(bf16_bits_to_f32(v[e]) * a.scale_log2,
                                        bf16_bits_to_f32(v[e + 1]) * a.scale_log2);
        v[e] = (uint16_t)(pr & 0xffffu);
        v[e + 1] = (uint16_t)(pr >> 16);
      }
      S.qpe[kk] = v;
    }
    S.qs *= a.scale_log2;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sref = fmaxf(sref, __shfl_xor(sref, m, 64));
    if (!(sref > 0.f)) sref = 1.f;
    inv_sref = 1.0f / sref;
    sref_256 = sref * (1.0f / 256.0f);
    S.qs *= sref;
  }
  barrier();
#pragma unroll
  for (int i = 2; i <= AHEAD; ++i) issue_tile(copy_of(k0 + i, i), w, lane);

  long p0, p1;
  f32x16 sl, sr;
  tile_step<true, false, false>(S, 0, 0, 0, 0, lane, lo, TileCopy{}, w, 0.f, sl, sr);
  tile_probs(a, S, sl, sr, stage_base(0), k0 * kTile, w, lane, inv_sref, sref_256, true, 0.f,
             p0, p1);
  const float shift = kShift - (S.m == -INFINITY ? INFINITY : S.m);
  for (int i = 1; i < n; ++i) {
    wait_vm<(AHEAD - 1) * kDma>();
    barrier();
    const int st = i % NSTAGE;
    const TileCopy c = copy_of(k0 + i + AHEAD, (i + AHEAD) % NSTAGE);
    tile_step<true, true, true>(S, st, (i - 1) % NSTAGE, p0, p1, lane, lo, c, w, shift, sl, sr);
    tile_probs(a, S, sl, sr, stage_base(st), (k0 + i) * kTile, w, lane, inv_sref, sref_256,
               false, shift, p0, p1);
  }
  tile_step<false, true, false>(S, 0, (n - 1) % NSTAGE, p0, p1, lane, lo, TileCopy{}, w, 0.f, sl,
                                sr);
  // (the last re-reads must land before the stages are reused or the
  // workgroup ends)
  wait_vm<0>();
}

// The chunk's partial: o~ / l (bf16) and its natural-log log-sum-exp, the
// rows staged in the idle ring so that they leave as whole 1 KiB rows.
constexpr int O_PITCH = D_LAT * 2 + 16;
static_assert(NW * 32 * O_PITCH <= NSTAGE * STAGE, "the staged rows fit the ring");

__device__ __forceinline__ void write_partial(const DecodeArgs& a, const State& S, int64_t slot,
                                              float sref_256, int w, int lane) {
  const int lc = lane & 31, hh = lane >> 5;
  mfma_drain();
  const float lsum = wave_sum_xor(S.l, 32);
  const int row = w * 32 + lc;
  if (hh == 0) a.part_lse[slot * kRowsPerWG + row] =
      lsum > 0.f ? (S.m + __log2f(lsum)) * kLn2 : -INFINITY;
  const float f = lsum > 0.f ? sref_256 / lsum : 0.f;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  MLA_LDS uint8_t* st = (MLA_LDS uint8_t*)s_ring + w * 32 * O_PITCH;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& v = S.o[db];
      *(MLA_LDS u32x2*)(st + lc * O_PITCH + (db * 32 + 8 * g + 4 * hh) * 2) =
          u32x2{pack_bf16x2(v[4 * g] * f, v[4 * g + 1] * f),
                pack_bf16x2(v[4 * g + 2] * f, v[4 * g + 3] * f)};
    }
  uint8_t* dst = (uint8_t*)a.part_o + (slot * kRowsPerWG + w * 32) * (D_LAT * 2) + lane * 16;
#pragma unroll
  for (int r = 0; r < 32; ++r)
    *(u32x4*)(dst + r * (D_LAT * 2)) = *(const MLA_LDS u32x4*)(st + r * O_PITCH + lane * 16);
}

__global__ __launch_bounds__(kThreads, 1) void decode_fp8_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const int lc = lane & 31, hh = lane >> 5;

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

  // query rows: row R = rg*128 + 32w + lc; lane (hh, lc) holds bytes
  // 64ks + 32hh .. +31 of its e4m3 row and dims 16k + 8hh .. +7 of q_pe
  const int rows_total = a.q_len * a.n_heads;
  const int R = ch.rg * kRowsPerWG + w * 32 + lc;
  const bool valid = R < rows_total;
  const int j = valid ? R / a.n_heads : 0;
  const int h = valid ? R % a.n_heads : 0;
  const int64_t qrow = ((int64_t)ch.b * a.q_len + j) * a.n_heads + h;
  State S;
#pragma unroll
  for (int db = 0; db < DB; ++db) S.o[db] = f32x16{};
  S.m = -INFINITY;
  S.l = 0.f;
  S.lim = valid ? (a.causal ? ch.len - a.q_len + j + 1 : ch.len) : 0;
  S.tmax = -INFINITY;
  S.redo = false;
  S.len = ch.len;
  auto load_query = [&]() {
    // (a row past the end reads row 0; its limit 0 masks every key)
    const uint8_t* q8 = (const uint8_t*)a.q_lat + qrow * D_LAT;
    const uint16_t* qpe = (const uint16_t*)a.q_pe + qrow * D_ROPE;
#pragma unroll
    for (int kk = 0; kk < KS_LAT; ++kk) S.q8[kk] = *(const i32x8*)(q8 + kk * 64 + hh * 32);
#pragma unroll
    for (int kk = 0; kk < KS_ROPE; ++kk) S.qpe[kk] = *(const u16x8*)(qpe + kk * 16 + hh * 8);
    S.qs = a.q_scale[qrow];
  };

  float inv_sref, sref_256;
  run_pass<true>(a, S, ch, k0, n, w, lane, load_query, inv_sref, sref_256);

  // rare second pass, with the true row maxima as references, when any row
  // of the workgroup saw a score past its reference + kSlack
  if (lane == 0) s_flag[w] = S.redo ? 1 : 0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  const bool any_redo = __ballot(lane < NW && s_flag[lane & (NW - 1)] != 0) != 0;
  if (any_redo) {
    S.m = wave_max_xor(S.tmax, 32);
    S.l = 0.f;
    mfma_drain();
#pragma unroll
    for (int db = 0; db < DB; ++db) S.o[db] = f32x16{};
    // (the pass's first copies go into stages 0 and 1: the barrier above
    // follows every wave's last read of them)
    run_pass<false>(a, S, ch, k0, n, w, lane, [] {}, inv_sref, sref_256);
  }
  write_partial(a, S, slot, sref_256, w, lane);
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
