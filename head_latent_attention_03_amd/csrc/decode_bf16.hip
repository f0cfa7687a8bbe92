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
// Mapping onto CDNA4 (4 waves, one per SIMD, 512 registers each):
//   * Wave w owns rows 32w .. 32w+31 outright: its absorbed query [32 x 576]
//     bf16 (144 VGPRs) and its output accumulator [32 x 512] f32 (256
//     registers, the accumulation file) stay resident for the whole chunk.
//   * Both products use v_mfma_f32_32x32x16_bf16.  Against 16x16 blocks this
//     halves the LDS bytes per flop of the operand that comes from LDS: a
//     CU's four SIMDs at full MFMA rate then need 128 B/clk of LDS reads,
//     where 16x16 blocks need 256 B/clk, more than the LDS delivers.
//   * S^T = K Q^T: A = 32 K rows x 16 dims from LDS (one ds_read_b128 per
//     lane), B = the query from registers.  The accumulator leaves lane l
//     with head l & 31 and 16 tokens, 8(i >> 2) + 4(l >> 5) + (i & 3): the
//     probabilities are already the B operand of the output product (lane =
//     one head, 8 tokens per 16-token k-step), so they never touch LDS.
//   * O^T += C^T P^T: A = 32 latent dims x 16 tokens, two ds_read_b64_tr_b16
//     (the LDS transpose read) per lane, with the tokens in the order the
//     score accumulator holds them.
//   * Iteration i copies tile i + 2, runs the output product of tile i - 1
//     and the scores of tile i with their MFMAs alternating (independent
//     accumulators, so the score chain never waits on its own latency), and
//     then the softmax of tile i.
//   * The 32-token tile [c ; k^R] (32 x 1152 B) is brought from HBM straight
//     into LDS with 16-byte global_load_lds (no VGPR staging), through a ring
//     of 4 stages: iteration i reads stages i - 1 (output) and i (scores),
//     tile i + 1 is in flight and tile i + 2 is copied into the stage that
//     tile i - 2 released.  Each wave copies 8 latent rows and the 8 rotary
//     rows of the same tokens per tile (9 instructions).  A sequence's page
//     numbers sit one per lane in a VGPR and are read with v_readlane.
//   * Online softmax in fp32 (base 2, scale folded).  Each row keeps a fixed
//     reference maximum, set by its first scores, instead of rescaling the
//     accumulator whenever the maximum grows, so the accumulator is only
//     ever written by MFMAs.  If a score passes m_ref + 64 the workgroup runs
//     its chunk once more with the true row maxima.
//   * LDS layout, for gfx950's LDS (64 banks of 4 bytes; a 16-byte read
//     serves its 64 lanes in four 16-lane cycles, lanes taken in quads: the
//     cycle of lane l is (l >> 5, parity of bits 2..4 of l); an 8-byte
//     transpose read serves lanes 0-31, then 32-63).  Latent row t is padded,
//     at t * 1088 + 16 ((t >> 2) & 3), so its 16-byte chunk c falls in slot
//     (4t + ((t >> 2) & 3) + c) mod 16 of a 256-byte bank span:
//       - QK: a cycle's 16 lanes read one chunk of 16 tokens 4a + r whose a
//         share a parity; (r, a & 3) takes each of its 16 values once;
//       - PV: a transpose half reads 4 consecutive chunks of 4 consecutive
//         tokens; 4(t & 3) spreads the tokens over the high two slot bits
//         while the chunks fill the low two;
//     and every latent read is one per-lane base plus an immediate.  Rotary
//     chunk c (0..7) of token t sits at c ^ rope_key(t), rope_key(t) =
//     ((t >> 2) & 3) + 4((t >> 1) & 1); with the row's 128-byte offset (bit 0
//     of t) it separates the 16 tokens of a QK cycle.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int D_LAT = 512;
constexpr int D_ROPE = 64;
constexpr int LAT_ROW = D_LAT * 2;         // bytes per cached latent row
constexpr int ROPE_ROW = D_ROPE * 2;       // bytes per cached rotary row
constexpr int KS_LAT = D_LAT / 16;         // QK k-steps over the latent
constexpr int KS_ROPE = D_ROPE / 16;       // QK k-steps over the rotary part
constexpr int KS = KS_LAT + KS_ROPE;       // 36
constexpr int DB = D_LAT / 32;             // 32-dim output blocks
constexpr int PV_STEPS = 2 * DB;           // two 16-token k-steps per tile
constexpr int LAT_PITCH = LAT_ROW + 64;      // LDS pitch of a latent row
constexpr int LAT_STAGE = kTile * LAT_PITCH; // 34 KiB
constexpr int ROPE_STAGE = kTile * ROPE_ROW; // 4 KiB
constexpr int STAGE = LAT_STAGE + ROPE_STAGE;
constexpr int NSTAGE = 4;
constexpr float kRefSlack = 64.0f;         // log2 units

constexpr int NW = kRowsPerWG / 32;        // 4 waves
constexpr int kThreads = 64 * NW;
constexpr int kLatRows = kTile / NW;       // latent rows each wave copies per tile (8)
constexpr int kDma = kLatRows + 1;         // copies per wave per tile
constexpr int kDmaEvery = 4;               // MFMA steps between a wave's copies

__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];
__shared__ int s_flag[NW];
static_assert(NSTAGE * STAGE + NW * 4 <= 160 * 1024, "LDS budget");

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// acc += A B with the accumulator pinned to the accumulation registers.  The
// 256 of them hold exactly the wave's output [32 x 512]; left to itself the
// allocator also places the score accumulator there and then moves an output
// block between register files every tile.  Each output block is updated by
// MFMAs only, at least 15 MFMAs apart; mfma_drain() covers the MFMA latency
// before anything else reads or writes the accumulators.
__device__ __forceinline__ void mfma32_acc(f32x16& acc, u16x8 a, u16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// LDS byte offset of latent row t within a stage, and the rotary swizzle key
// (see the header)
__host__ __device__ constexpr int lat_row(int t) { return t * LAT_PITCH + 16 * ((t >> 2) & 3); }
__device__ __forceinline__ int rope_key(int t) { return ((t >> 2) & 3) | (((t >> 1) & 1) << 2); }
static_assert(lat_row(kTile - 1) + LAT_ROW <= LAT_STAGE, "latent rows fit the stage");

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

// The copies of one tile: wave w's latent rows 8w .. 8w+7 (parts 0..7, one
// 1 KiB row each) and the rotary rows of the same tokens (part 8).  Tokens
// past the end of the sequence re-read its last token (finite data that the
// mask then ignores), so every wave issues the same count.
struct TileCopy {
  const uint8_t* lat;    // first latent row of the tile
  const uint8_t* rope;   // first rotary row of the tile
  int tok0, last;        // first token of the tile, last token of the sequence
  int st;                // ring stage
};

__device__ __forceinline__ TileCopy tile_copy(const DecodeArgs& a, int page, int len, int k,
                                              int st) {
  TileCopy c;
  c.tok0 = k * kTile;
  c.last = len - 1;
  const int64_t row0 = (int64_t)page * kPage + (c.tok0 % kPage);
  c.lat = (const uint8_t*)a.kv_lat + row0 * LAT_ROW;
  c.rope = (const uint8_t*)a.kv_rope + row0 * ROPE_ROW;
  c.st = st;
  return c;
}

__device__ __forceinline__ void issue_part(const TileCopy& c, int j, int w, int lane) {
  static_assert(kLatRows * ROPE_ROW == 1024, "a wave's rotary rows fill one 1 KiB copy");
  MLA_LDS uint8_t* dst = stage_base(c.st);
  if (j < kLatRows) {
    // one row, copied as it is: lane l brings chunk l
    const int t = w * kLatRows + j;
    const int tc = min(c.tok0 + t, c.last) - c.tok0;
    dma16_s(c.lat + tc * LAT_ROW, (uint32_t)(lane << 4), dst + lat_row(t));
  } else {
    const int t = w * kLatRows + (lane >> 3);
    const int tc = min(c.tok0 + t, c.last) - c.tok0;
    const uint32_t off = (uint32_t)(tc * ROPE_ROW + (((lane & 7) ^ rope_key(t)) << 4));
    dma16_s(c.rope, off, dst + LAT_STAGE + w * kLatRows * ROPE_ROW);
  }
}

// Entries pg and pg + 1 of a block-table row (clamped to its max_pages
// entries) by scalar loads, waited for in place.  The wait counts scalar
// loads only: it neither holds on the vector loads in flight nor leaves the
// compiler a vector load to wait for, whose wait would count every older
// vector load and copy (so that the first tiles' copies would go out one tile
// at a time).  glc reads from L2, past the scalar cache, so no line cached
// there before the table was last written can be seen.
__device__ __forceinline__ void scalar_table_entries2(const int32_t* row, int pg, int max_pages,
                                                      int (&out)[2]) {
  const int32_t* p0 = row + min(pg, max_pages - 1);
  const int32_t* p1 = row + min(pg + 1, max_pages - 1);
  int v0, v1;
  asm volatile("s_load_dword %0, %2, 0x0 glc\n\ts_load_dword %1, %3, 0x0 glc\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1)
               : "s"(p0), "s"(p1)
               : "memory");
  out[0] = v0;
  out[1] = v1;
}

__device__ __forceinline__ void issue_tile(const TileCopy& c, int w, int lane) {
#pragma unroll
  for (int j = 0; j < kDma; ++j) issue_part(c, j, w, lane);
}

// The copies of a tile wholly inside the sequence (non-temporal, as every
// cache copy of the decode), with no per-copy address
// arithmetic: the wave's latent row 8w + j of the tile is base + j KiB, read
// as base (j < 4) or base + 4 KiB (j >= 4) plus an instruction offset of
// (j & 3) KiB, and it lands at stage + lat_row(8w + j) = stage + lat_row(8w)
// + 1088 j + 16 (j >> 2) (for w < 4).  The instruction offset moves the LDS
// destination too (M0 + offset + 16 lane), so M0 is set that much lower.
struct FastCopy {
  const uint8_t* lat;    // latent row 8w of the tile
  const uint8_t* lat4;   // latent row 8w + 4
  const uint8_t* rope;   // rotary row 0 of the tile
  uint32_t m0_lat;       // LDS address of row 8w in the stage
  uint32_t m0_rope;      // LDS address of the wave's rotary rows in the stage
};

struct FastLane {
  uint32_t lat;          // lane * 16
  uint32_t rope;         // rotary offset of the lane's chunk (see issue_part)
};

__device__ __forceinline__ constexpr uint32_t lat_row_j(int j) { return 1088u * j + 16u * (j >> 2); }
static_assert(LAT_PITCH == 1088, "lat_row_j assumes the 1088-byte pitch");

__device__ __forceinline__ FastCopy fast_copy(const DecodeArgs& a, int page, int k, int st, int w) {
  FastCopy c;
  const int64_t row0 = (int64_t)page * kPage + ((k * kTile) % kPage);
  c.lat = (const uint8_t*)a.kv_lat + (row0 + 8 * w) * LAT_ROW;
  c.lat4 = c.lat + 4 * LAT_ROW;
  c.rope = (const uint8_t*)a.kv_rope + row0 * ROPE_ROW;
  const uint32_t sb = (uint32_t)(uintptr_t)stage_base(st);
  c.m0_lat = uni(sb + lat_row(8 * w));
  c.m0_rope = uni(sb + LAT_STAGE + w * kLatRows * ROPE_ROW);
  return c;
}

template <int J>
__device__ __forceinline__ void issue_fast(const FastCopy& c, const FastLane& fl) {
  if constexpr (J < kLatRows) {
    constexpr int off = (J & 3) * LAT_ROW;
    constexpr uint32_t m0_add = lat_row_j(J) - (uint32_t)off;
    const uint8_t* base = J < 4 ? c.lat : c.lat4;
    asm volatile("s_add_u32 m0, %0, %1\n\tglobal_load_lds_dwordx4 %2, %3 offset:%4 nt"
                 :
                 : "s"(c.m0_lat), "i"(m0_add), "v"(fl.lat), "s"(base), "i"(off)
                 : "memory", "m0", "scc");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(c.m0_rope), "v"(fl.rope), "s"(c.rope)
                 : "memory", "m0");
  }
}

template <int J = 0>
__device__ __forceinline__ void issue_fast_part(const FastCopy& c, const FastLane& fl, int j) {
  if constexpr (J < kDma) {
    if (j == J) issue_fast<J>(c, fl);
    else issue_fast_part<J + 1>(c, fl, j);
  }
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
  u16x8 q[KS];          // absorbed query of the wave's rows (B operand)
  f32x16 o[DB];         // O^T accumulator: lane holds head l & 31 and 16 of
                        // the block's 32 latent dims
  float m, l;           // reference max (log2 units, scaled) and per-lane sum
  int lim;              // keys visible to the lane's row: t < lim
  float tmax;           // largest score this lane has seen (log2 units, scaled)
  bool redo;            // a score passed m_ref + 64 with mass already accumulated
};

// Per-lane LDS byte offsets of the read patterns (from a stage's base).  The
// latent reads are one of them plus an immediate:
//   QK latent, k-step ks:   qk + 32 ks
//   QK rotary, k-step 32+k: rp ^ (2k << 4)
//   PV block db, k-step kb, read r (tokens +8r):
//                           pv + LAT_PITCH (16kb + 8r) + 32r + 64db
// (lat_row(t0 + t) = lat_row(t) + LAT_PITCH t0 + 32 (t0 >> 3 & 1) for t0 a
// multiple of 8 and t < 8).
struct LaneOff {
  uint32_t qk, rp, pv;
};

__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int lc = lane & 31, hh = lane >> 5;
  const int dh = (lane >> 4) & 1, lr = lane & 15;
  LaneOff o;
  // QK: lane reads token lc, chunk 2ks + hh
  o.qk = (uint32_t)(lat_row(lc) + 16 * hh);
  o.rp = (uint32_t)(LAT_STAGE + lc * ROPE_ROW + ((hh ^ rope_key(lc)) << 4));
  // PV transpose read: lane addresses token 4hh + (lr >> 2) (+16kb + 8r) and
  // latent dims 32db + 16dh + 4(lr & 3) .. +3: chunk 4db + 2dh + ((lr & 3) >> 1),
  // byte 8 (lr & 1)
  o.pv = (uint32_t)(lat_row(4 * hh + (lr >> 2)) + 16 * (2 * dh + ((lr & 3) >> 1)) + 8 * (lr & 1));
  return o;
}

// A operand of score k-step ks (K rows of tile stage kq), and of output step
// j: k-step kb = j >> 4 (tokens 16kb ..), block db = j & 15 (C^T of stage kv)
__device__ __forceinline__ u16x8 load_k(const MLA_LDS uint8_t* kq, const LaneOff& lo, int ks) {
  if (ks < KS_LAT) return *(const MLA_LDS u16x8*)(kq + lo.qk + 32 * ks);
  return *(const MLA_LDS u16x8*)(kq + (lo.rp ^ (uint32_t)((2 * (ks - KS_LAT)) << 4)));
}

__device__ __forceinline__ u16x8 load_v(const MLA_LDS uint8_t* kv, const LaneOff& lo, int j) {
  const int kb = j >> 4, db = j & 15;
  const MLA_LDS uint8_t* b = kv + lo.pv + 16 * kb * LAT_PITCH + 64 * db;
  const u16x4 lo4 = lds_read_tr16(b);
  const u16x4 hi4 = lds_read_tr16(b + 8 * LAT_PITCH + 32);
  return u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
}

// LDS reads run this many MFMA steps ahead of their use
constexpr int AH = 2;

// One pipeline step group: the scores of tile stage st_qk (if QK) and the
// output product of tile stage st_pv with probabilities p (if PV), issued
// alternately, plus the copies of a later tile (cp), one every kDmaEvery
// steps.  A copy instruction holds its wave for some 50 cycles; issued ahead
// of a step's MFMAs, part of that hides behind the MFMA still running.
template <bool QK, bool PV, bool COPY, bool FAST = false>
__device__ __forceinline__ void tile_step(State& S, int st_qk, int st_pv, const u16x8 (&p)[2],
                                          int lane, LaneOff lo, const TileCopy& cp, int w,
                                          f32x16& sacc, const FastCopy& fc = FastCopy{},
                                          const FastLane& fl = FastLane{}) {
  constexpr int NSTEP = QK ? KS : PV_STEPS;
  static_assert(kDmaEvery * (kDma - 1) + kDmaEvery - 1 < KS, "a tile's copies fit in the score steps");
  const MLA_LDS uint8_t* kq = stage_base(st_qk);
  const MLA_LDS uint8_t* kv = stage_base(st_pv);
  asm volatile("" : "+v"(lo.qk), "+v"(lo.rp), "+v"(lo.pv));
  u16x8 ka[AH], va[AH];
  if (QK) sacc = f32x16{};
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    if (QK) ka[j] = load_k(kq, lo, j);
    if (PV) va[j] = load_v(kv, lo, j);
  }
#pragma unroll
  for (int j = 0; j < NSTEP; ++j) {
    // a copy is issued while the previous step's MFMA still runs
    if (COPY && j % kDmaEvery == 0 && j / kDmaEvery < kDma) {
      if (FAST)
        issue_fast_part(fc, fl, j / kDmaEvery);
      else
        issue_part(cp, j / kDmaEvery, w, lane);
    }
    if (QK) {
      const u16x8 cur = ka[j % AH];
      if (j + AH < KS) ka[j % AH] = load_k(kq, lo, j + AH);
      sacc = mfma32(cur, S.q[j], sacc);
    }
    if (PV && j < PV_STEPS) {
      const u16x8 cur = va[j % AH];
      if (j + AH < PV_STEPS) va[j % AH] = load_v(kv, lo, j + AH);
      mfma32_acc(S.o[j & (DB - 1)], cur, p[j >> 4]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The probabilities of the later tiles packed as bf16 pairs (see above); with
// MASK, keys at or past the row's limit are cut.
template <bool MASK>
__device__ __forceinline__ void later_probs(const DecodeArgs& a, State& S, const f32x16& sacc,
                                            int tok0, int hh, uint32_t (&pk)[8]) {
  const float m_eff = S.m == -INFINITY ? INFINITY : S.m;
  float d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) d[i] = fmaf(sacc[i], a.scale_log2, -m_eff);
  if (MASK && __ballot(tok0 + kTile > S.lim)) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tok0 + 8 * (i >> 2) + 4 * hh + (i & 3) >= S.lim) d[i] = -INFINITY;
  }
  float dmx = d[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) dmx = fmaxf(dmx, d[i]);
  // (a row without reference gives -inf + inf = NaN, which fmaxf ignores)
  S.tmax = fmaxf(S.tmax, dmx + m_eff);
  S.redo |= dmx > kRefSlack;
  // (a probability past 2^64 only occurs in a pass that is redone, which
  // clears the accumulator and the sum; up to 2^128 it stays finite)
#pragma unroll
  for (int c = 0; c < 8; ++c)
    pk[c] = pack_bf16x2(fast_exp2(d[2 * c]), fast_exp2(d[2 * c + 1]));
}

// Adds the rounded probabilities to the lane's sum (v_dot2 with ones, so the
// sum sees the values the MFMA multiplies) and forms the two B operands.
__device__ __forceinline__ void finish_probs(State& S, const uint32_t (&pk)[8], u16x8 (&pout)[2]) {
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  float psum = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[c]), one2, psum, false);
  S.l += psum;
  pout[0] = __builtin_bit_cast(u16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
  pout[1] = __builtin_bit_cast(u16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
}

// Online softmax of a tile, in two parts.  Lane holds head l & 31 and tokens
// 8(i >> 2) + 4hh + (i & 3) of the tile.
//   * set_reference (the chunk's first tile only): a row's first scores set
//     its reference, formed across the row's two lanes.
//   * probs: every row with a visible key in the chunk has its reference by
//     then (the first tile holds the chunk's first key, and visibility is a
//     prefix), so d = s - m is one FMA per score, a jump past the reference
//     + 64 is one compare per tile (it marks the workgroup for a second
//     pass), and masking is needed only on a tile that crosses some row's
//     limit.  A row with no reference has no visible key: its d is -inf (m
//     taken as +inf).
__device__ __forceinline__ void set_reference(const DecodeArgs& a, State& S, const f32x16& sacc,
                                              int tok0, int lane) {
  const int hh = lane >> 5;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tok0 + 8 * (i >> 2) + 4 * hh + (i & 3);
    mx = fmaxf(mx, (t < S.lim) ? sacc[i] * a.scale_log2 : -INFINITY);
  }
  if (__ballot(mx > S.m + kRefSlack)) {
    mx = wave_max_xor(mx, 32);
    const float mass = wave_sum_xor(S.l, 32);
    if (mx > S.m + kRefSlack && mass == 0.f) S.m = mx;
  }
}

template <bool MASK>
__device__ __forceinline__ void probs(const DecodeArgs& a, State& S, const f32x16& sacc, int tok0,
                                      int lane, u16x8 (&pout)[2]) {
  uint32_t pk[8];
  later_probs<MASK>(a, S, sacc, tok0, lane >> 5, pk);
  finish_probs(S, pk, pout);
}


// One pass over the chunk's tiles [k0, k0 + n).  Iteration i (0 <= i <= n)
// runs the output product of tile i - 1 and the scores of tile i.
// The pass starts by calling `loads`, which issues NLOADS vector loads (the
// query, on the first pass) right after the block-table read, so that their
// latency overlaps that read's; then it copies tiles 0 and 1.  Tile 0 is
// waited for alone, and the loads, issued before it, have landed with it
// (the compiler's own waits for their registers can still count tile 1's
// copies, which are younger, but those land right behind tile 0's).  Tile 2
// is copied after the first scores.
template <int NLOADS, typename Loads>
__device__ __forceinline__ void run_pass(const DecodeArgs& a, State& S, const Chunk& ch, int k0,
                                         int n, int w, int lane, Loads loads) {
  const LaneOff lo = lane_offsets(lane);
  const int32_t* bt_row = a.block_table + (int64_t)ch.b * a.max_pages;
  PageWindow W;
  W.pg0 = uni(k0 * kTile / kPage);
  // every iteration copies one tile, so that the copy count (and with it each
  // vmcnt wait) is the same on every path; a copy past the chunk's last tile
  // re-reads that tile into a stage that is not read again
  const int k_last = k0 + n - 1;
  auto copy_of = [&](int k, int st) {
    k = min(k, k_last);
    const int page = page_lookup(W, bt_row, a.max_pages, k * kTile / kPage, lane);
    return tile_copy(a, page, ch.len, k, st);
  };
  // the first tiles' pages by scalar loads (tiles 0 .. 2 lie in
  // pages pg0 and pg0 + 1), then the page window of the later tiles
  static_assert(kPage == 2 * kTile, "tiles 0 .. 2 lie in two pages");
  loads();
  int pgs[2];
  scalar_table_entries2(bt_row, W.pg0, a.max_pages, pgs);
  auto prologue_copy = [&](int k, int st) {
    k = min(k, k_last);
    const int page = uni(k * kTile / kPage - W.pg0) == 0 ? pgs[0] : pgs[1];
    return tile_copy(a, page, ch.len, k, st);
  };
  issue_tile(prologue_copy(k0, 0), w, lane);
  issue_tile(prologue_copy(k0 + 1, 1), w, lane);
  W.v = page_window_load(bt_row, a.max_pages, W.pg0, lane);
  wait_vm<kDma + 1>();
  barrier();

  // Iteration i (1 <= i < n) waits for tile i (this wave's copies are done
  // once at most kDma newer ones, tile i + 1's, are outstanding; after the
  // barrier every wave's are, and every wave is done with stage (i - 2) & 3),
  // copies tile i + 2, runs the output product of tile i - 1 beside the
  // scores of tile i, and then the softmax of tile i.
  u16x8 p[2];
  f32x16 sacc;
  tile_step<true, false, false>(S, 0, 0, p, lane, lo, TileCopy{}, w, sacc);
  // (the page window is needed from iteration 1 on: waiting for it here, with
  // tile 1, keeps the compiler's wait out of the loop, where it would count
  // the copies of later tiles)
  asm volatile("" ::"v"(W.v));
  issue_tile(prologue_copy(k0 + 2, 2), w, lane);
  set_reference(a, S, sacc, k0 * kTile, lane);
  probs<true>(a, S, sacc, k0 * kTile, lane, p);
  // Iterations 1 .. n_fast - 1 take the fast path: their tile has no key at
  // or past any row's limit (no mask: the smallest limit of the rows is
  // L - q_len + 1 with the causal rule, L without), and the tile they copy
  // lies wholly inside the sequence (no clamped rows, so every copy address
  // is a tile base plus loop-invariant offsets).
  const int lim_min = a.causal ? ch.len - a.q_len + 1 : ch.len;
  const int mask_free = lim_min >= kTile ? lim_min / kTile - k0 : 0;   // i < mask_free
  const int copy_free = (k_last + 1) * kTile <= ch.len ? n : n - 3;    // i < copy_free
  const int n_fast = max(1, min(n, min(mask_free, copy_free)));
  FastLane fl;
  fl.lat = (uint32_t)lane << 4;
  {
    const int t = w * kLatRows + (lane >> 3);
    fl.rope = (uint32_t)(t * ROPE_ROW + (((lane & 7) ^ rope_key(t)) << 4));
  }
  int i = 1;
  for (; i < n_fast; ++i) {
    wait_vm<kDma>();
    barrier();
    const int kc = min(k0 + i + 2, k_last);
    const int page = page_lookup(W, bt_row, a.max_pages, kc * kTile / kPage, lane);
    const FastCopy fc = fast_copy(a, page, kc, (i + 2) & 3, w);
    tile_step<true, true, true, true>(S, i & 3, (i - 1) & 3, p, lane, lo, TileCopy{}, w, sacc,
                                      fc, fl);
    probs<false>(a, S, sacc, (k0 + i) * kTile, lane, p);
  }
  for (; i < n; ++i) {
    wait_vm<kDma>();
    barrier();
    const TileCopy c = copy_of(k0 + i + 2, (i + 2) & 3);
    tile_step<true, true, true>(S, i & 3, (i - 1) & 3, p, lane, lo, c, w, sacc);
    probs<true>(a, S, sacc, (k0 + i) * kTile, lane, p);
  }
  tile_step<false, true, false>(S, 0, (n - 1) & 3, p, lane, lo, TileCopy{}, w, sacc);
  // (the last re-reads must land before the stages are reused or the
  // workgroup ends)
  wait_vm<0>();
}

// The chunk's partial: o~ / l (rounded to bf16, like the output it feeds)
// and its natural-log log-sum-exp.  A row's sum is split over its two lanes.
// The accumulator layout gives each lane 8-byte pieces of one row, so a
// direct store would write 16 bytes of each of 32 rows per instruction; the
// rows are staged in the (by then idle) ring instead and leave as whole
// 1 KiB rows, one per store instruction.
constexpr int O_PITCH = D_LAT * 2 + 16;   // LDS pitch of a staged output row
static_assert(NW * 32 * O_PITCH <= NSTAGE * STAGE, "the staged rows fit the ring");

__device__ __forceinline__ void write_partial(const DecodeArgs& a, const State& S, int64_t slot,
                                              int w, int lane) {
  const int lc = lane & 31, hh = lane >> 5;
  mfma_drain();
  const float lsum = wave_sum_xor(S.l, 32);
  const int row = w * 32 + lc;
  if (hh == 0) a.part_lse[slot * kRowsPerWG + row] =
      lsum > 0.f ? (S.m + __log2f(lsum)) * kLn2 : -INFINITY;
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  // every wave is done with the ring once all have passed this barrier
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  MLA_LDS uint8_t* st = (MLA_LDS uint8_t*)s_ring + w * 32 * O_PITCH;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& v = S.o[db];
      *(MLA_LDS u32x2*)(st + lc * O_PITCH + (db * 32 + 8 * g + 4 * hh) * 2) =
          u32x2{pack_bf16x2(v[4 * g] * inv, v[4 * g + 1] * inv),
                pack_bf16x2(v[4 * g + 2] * inv, v[4 * g + 3] * inv)};
    }
  // (each wave reads back only its own rows)
  uint8_t* dst = (uint8_t*)a.part_o + (slot * kRowsPerWG + w * 32) * (D_LAT * 2) + lane * 16;
#pragma unroll
  for (int r = 0; r < 32; ++r)
    *(u32x4*)(dst + r * (D_LAT * 2)) = *(const MLA_LDS u32x4*)(st + r * O_PITCH + lane * 16);
}

__global__ __launch_bounds__(kThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const int lc = lane & 31, hh = lane >> 5;

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
  const int n = k1 - k0;
  const int64_t slot = g;

  // query rows of this unit; the (query, head) row of lane (hh, lc) is
  // R = rg*128 + 32w + lc
  const int rows_total = a.q_len * a.n_heads;
  const uint16_t* qlat = (const uint16_t*)a.q_lat;
  const uint16_t* qpe = (const uint16_t*)a.q_pe;
  State S;
  const int R = ch.rg * kRowsPerWG + w * 32 + lc;
  const bool valid = R < rows_total;
  const int jq = valid ? R / a.n_heads : 0;
  const int hq = valid ? R % a.n_heads : 0;
#pragma unroll
  for (int db = 0; db < DB; ++db) S.o[db] = f32x16{};
  S.m = -INFINITY;
  S.l = 0.f;
  S.lim = valid ? (a.causal ? ch.len - a.q_len + jq + 1 : ch.len) : 0;
  S.tmax = -INFINITY;
  S.redo = false;
  // the query (KS vector loads per lane, issued right after the block-table
  // read); lane (hh, lc) holds dims 16ks + 8hh .. +7 of its row for every
  // k-step ks
  auto load_query = [&]() {
    const int64_t qrow = ((int64_t)ch.b * a.q_len + jq) * a.n_heads + hq;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u16x8 v;
      if (kk < KS_LAT)
        v = *(const u16x8*)(qlat + qrow * D_LAT + kk * 16 + hh * 8);
      else
        v = *(const u16x8*)(qpe + qrow * D_ROPE + (kk - KS_LAT) * 16 + hh * 8);
      S.q[kk] = v;   // (a row past the end reads row 0; its limit 0 masks every key)
    }
  };

  run_pass<KS>(a, S, ch, k0, n, w, lane, load_query);

  // rare second pass, with the true row maxima as references, when any row
  // of the workgroup saw a score jump; every wave posts its flag
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
    run_pass<0>(a, S, ch, k0, n, w, lane, [] {});
  }
  write_partial(a, S, slot, w, lane);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_bf16_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
