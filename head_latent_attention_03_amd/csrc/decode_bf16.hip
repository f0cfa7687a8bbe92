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
// Mapping onto CDNA4 (8 waves, two per SIMD):
//   * Scores: wave w owns rows 16w .. 16w+15; its absorbed query [16 x 576]
//     bf16 stays in VGPRs.  Output: waves 2p and 2p+1 share rows 32p .. 32p+31
//     and each accumulates half of the 512 latent columns for both row
//     blocks ([32 x 256] f32 in registers), so every C^T block read from LDS
//     feeds two MFMAs.  The pair swaps probabilities through LDS (1 KiB per
//     wave and tile).  Per tile, LDS serves the score operand eight times
//     (8 x 36 KiB) but the value operand four times (8 x 16 KiB), against
//     eight times (8 x 32 KiB) when every wave holds whole rows.
//   * The output product of tile i runs one iteration after its scores, so
//     the probabilities a wave stores in iteration i are read by its partner
//     in iteration i + 1, behind the one barrier every iteration has; they are
//     double-buffered by tile parity.
//   * The 32-token tile [c ; k^R] (32 x 1152 B) is brought from HBM straight
//     into LDS with 16-byte global_load_lds (no VGPR staging), through a ring
//     of 4 stages: iteration i reads stages i - 1 (output) and i (scores),
//     tile i + 1 is in flight and tile i + 2 is copied into the stage that
//     tile i - 2 released.  A sequence's page numbers sit one per lane in a
//     VGPR and are read with v_readlane.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows from LDS
//     (ds_read_b128), B = the query from registers.  The accumulator leaves
//     each lane with one head and 8 tokens, exactly the B operand of the
//     output product, so the probabilities travel as one 16-byte chunk per
//     lane.
//   * O^T += C^T P^T with the same MFMA: A = C^T read with ds_read_b64_tr_b16
//     (the LDS transpose read), B = P from LDS.
//   * The HBM -> LDS copies are issued from inline asm (see dma16_s), so the
//     compiler schedules the LDS reads freely; the ring is guarded by explicit
//     vmcnt waits and one barrier per iteration.
//   * Online softmax in fp32 (base 2, scale folded).  Each row keeps a fixed
//     reference maximum, set by its first scores, instead of rescaling the
//     accumulator whenever the maximum grows: probabilities are
//     exp2(s - m_ref) <= 2^64, so nothing overflows, and no cross-lane
//     traffic is needed while scores stay below m_ref + 64.  If a score passes
//     that, the workgroup runs its chunk once more with the true row maxima.
//     The accumulator is thus only ever written by MFMAs, which is what lets
//     two waves share a row's columns.
//   * LDS rows are XOR-swizzled on 16-byte chunks so both read patterns are
//     bank-conflict free on gfx950's LDS (64 banks of 4 bytes; a 16-byte read
//     serves its 64 lanes in four 16-lane cycles, lanes taken in quads: the
//     cycle of lane l is (l >> 5, parity of bits 2..4 of l); an 8-byte
//     transpose read serves lanes 0-31, then 32-63).  Latent chunk c of token
//     t sits at c ^ lat_key(t), lat_key(t) = 2(t & 7) ^ 9[bit 3 of t]:
//       - QK: the 16 lanes of a cycle read chunk lg ^ lat_key(lr) for eight
//         tokens with one lg and eight with lg ^ 1; the two key sets are
//         unions of whole pairs {2m, 2m + 1} and fill all 16 chunk slots;
//       - PV: the 8 tokens of a transpose half have distinct lat_key >> 1, so
//         their 32-byte chunk pairs cover the 256-byte bank span once;
//       - the copies: lat_key(4w + j) = lat_key(4w) ^ 2j, one XOR per row.
//     Rotary chunk c sits at c ^ rope_key(t).  The probabilities are stored
//     lane-major (chunk g of row h at g * 2 KiB + 16 h), so the 16 lanes of a
//     cycle read 256 contiguous bytes.
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
constexpr int DB = D_LAT / 16;             // 16-column output blocks
constexpr int DBH = DB / 2;                // output column blocks per wave
constexpr int LAT_STAGE = kTile * LAT_ROW;   // 32 KiB
constexpr int ROPE_STAGE = kTile * ROPE_ROW; // 4 KiB
constexpr int STAGE = LAT_STAGE + ROPE_STAGE;
constexpr int NSTAGE = 4;
constexpr float kRefSlack = 64.0f;         // log2 units

constexpr int kWaves = kRowsPerWG / 16;    // 8
constexpr int kThreads = 64 * kWaves;
constexpr int kLatRows = kTile / kWaves;   // latent rows each wave copies per tile (4)
constexpr int kDma = kLatRows + 1;         // copies per wave per tile
constexpr int P_BUF = kRowsPerWG * kTile * 2;  // one tile's probabilities, bf16 (8 KiB)
constexpr int P_CHUNK = kRowsPerWG * 16;       // bytes per 16-byte chunk column (2 KiB)

// the ring and the two probability buffers fill the 160 KiB of LDS exactly;
// the few words needed after a pass (the second-pass flags, 1 / l) reuse the
// probability buffers once the pass is over
__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];
__shared__ __attribute__((aligned(1024))) uint8_t s_p[2 * P_BUF];
static_assert(NSTAGE * STAGE + 2 * P_BUF <= 160 * 1024, "LDS budget");

// swizzle keys (see the header); both depend on t & 15 only
__device__ __forceinline__ int lat_key(int t) { return ((t & 7) << 1) ^ (((t >> 3) & 1) * 9); }
__device__ __forceinline__ int rope_key(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

// The copies of one tile: this wave's kLatRows latent rows (parts
// 0..kLatRows-1) and the rotary rows of the same tokens (last part, on half
// the lanes).  Tokens past the end of the sequence re-read its last token
// (finite data that the mask then ignores), so every wave issues the same
// count.  The parts are issued along a phase's MFMA steps, so their issue
// (which waits while the memory pipeline is full) overlaps the MFMAs.
struct TileCopy {
  const uint8_t* lat;    // first latent row of the tile
  const uint8_t* rope;   // first rotary row of the tile
  int tok0, last;        // first token of the tile, last token of the sequence
  int st;                // ring stage
  bool valid;
};

__device__ __forceinline__ TileCopy tile_copy(const DecodeArgs& a, int page, int len, int k,
                                              int st, bool valid) {
  TileCopy c;
  c.tok0 = k * kTile;
  c.last = len - 1;
  const int64_t row0 = (int64_t)page * kPage + (c.tok0 % kPage);
  c.lat = (const uint8_t*)a.kv_lat + row0 * LAT_ROW;
  c.rope = (const uint8_t*)a.kv_rope + row0 * ROPE_ROW;
  c.st = st;
  c.valid = valid;
  return c;
}

__device__ __forceinline__ void issue_part(const TileCopy& c, int j, int w, int lane) {
  constexpr int NL = kLatRows;
  static_assert(NL * ROPE_ROW * 2 == 1024, "a wave's rotary rows fill half a 1 KiB copy");
  MLA_LDS uint8_t* dst = stage_base(c.st);
  if (j < NL) {
    // lat_key(w*NL + q) = lat_key(w*NL) ^ 2q for q < NL, so the source chunk
    // offsets of the wave's rows are one per-lane value XOR 32q
    uint32_t off0 = (uint32_t)((lane ^ lat_key(w * NL)) << 4);
    asm volatile("" : "+v"(off0));
    const int t = w * NL + j;
    const int tc = min(c.tok0 + t, c.last) - c.tok0;
    dma16_s(c.lat + tc * LAT_ROW, off0 ^ (uint32_t)(j << 5), dst + t * LAT_ROW);
  } else {
    const int t = w * NL + (lane >> 3);
    const int tc = min(c.tok0 + t, c.last) - c.tok0;
    const uint32_t off = (uint32_t)(tc * ROPE_ROW + (((lane & 7) ^ rope_key(t)) << 4));
    if (lane < NL * 8) dma16_s(c.rope, off, dst + LAT_STAGE + w * NL * ROPE_ROW);
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
  u16x8 q[KS];          // absorbed query of the wave's rows (B operand)
  f32x4 o[2][DBH];      // O^T accumulator of the pair's row block j and this
                        // wave's column block: lane holds head lr, 4 latent dims
  float m, l;           // reference max (log2 units, scaled) and per-lane sum
  int lim;              // keys visible to the lane's row: t < lim
  float tmax;           // largest score this lane has seen (log2 units, scaled)
  bool redo;            // a score passed m_ref + 64 with mass already accumulated
};

// Per-lane LDS byte offsets of the read patterns (from a stage's base, or
// from a probability buffer).  Every address a tile reads is one of them
// XOR or plus a small constant:
//   QK latent, chunk group v:  qk ^ (v << 6)   ((v*4 + lg) ^ key = (lg ^ key) ^ 4v)
//   QK rotary, chunk group v:  rp ^ (v << 6)
//   PV transpose, column db:   pv ^ ((db & 7) << 5), + 256 per 8 columns
//   probabilities of block rb: p + 256 rb
// (the bases are 1 KiB aligned and the XORed bits never carry).
struct LaneOff {
  uint32_t qk, rp, pv, p;
};

__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int t1 = lg * 4 + (lr >> 2);
  LaneOff o;
  o.qk = (uint32_t)(lr * LAT_ROW + ((lg ^ lat_key(lr)) << 4));
  o.rp = (uint32_t)(LAT_STAGE + lr * ROPE_ROW + ((lg ^ rope_key(lr)) << 4));
  o.pv = (uint32_t)(t1 * LAT_ROW + ((((lr & 3) >> 1) ^ lat_key(t1)) << 4) + ((lr & 1) << 3));
  o.p = (uint32_t)(lg * P_CHUNK + lr * 16);
  return o;
}

// ---- S^T[t, h] = K[t, :] . Q[h, :] for one tile (t = tb*16 + row of the
// 16x16 block).  Also issues the copy parts of a later tile (cp), one per two
// k-steps.
__device__ __forceinline__ void tile_qk(const State& S, int st, int lane, LaneOff lo,
                                        const TileCopy& cp, int w, f32x4 (&sacc)[2]) {
  static_assert(2 * kDma <= KS, "a tile's copies fit in the QK k-steps");
  const MLA_LDS uint8_t* lat = stage_base(st);
  asm volatile("" : "+v"(lo.qk), "+v"(lo.rp));
  sacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // latent chunk kk*4 + lg of token tb*16 + lr sits at ((kk & 3)*4 + lg) ^ key
  // within the 16-chunk group kk >> 2 (key < 16); rotary chunk k2*4 + lg at
  // (k2*4 + lg) ^ rope_key
  auto load_k = [&](int kk, int tb) -> u16x8 {
    if (kk < KS_LAT)
      return *(const MLA_LDS u16x8*)(lat + (lo.qk ^ (uint32_t)((kk & 3) << 6)) + tb * 16 * LAT_ROW +
                                     (kk >> 2) * 256);
    return *(const MLA_LDS u16x8*)(lat + (lo.rp ^ (uint32_t)((kk - KS_LAT) << 6)) +
                                   tb * 16 * ROPE_ROW);
  };
  // A operands are read QK_AHEAD k-steps ahead of their MFMAs
#ifdef MLA_QK_AHEAD
  constexpr int QK_AHEAD = MLA_QK_AHEAD;
#else
  constexpr int QK_AHEAD = 2;
#endif
  u16x8 ka[QK_AHEAD][2];
#pragma unroll
  for (int j = 0; j < QK_AHEAD; ++j) {
    ka[j][0] = load_k(j, 0);
    ka[j][1] = load_k(j, 1);
  }
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const u16x8 cur0 = ka[kk % QK_AHEAD][0], cur1 = ka[kk % QK_AHEAD][1];
    if (kk + QK_AHEAD < KS) {
      ka[kk % QK_AHEAD][0] = load_k(kk + QK_AHEAD, 0);
      ka[kk % QK_AHEAD][1] = load_k(kk + QK_AHEAD, 1);
    }
    sacc[0] = mfma_bf16_16x16x32(cur0, S.q[kk], sacc[0]);
    sacc[1] = mfma_bf16_16x16x32(cur1, S.q[kk], sacc[1]);
    if ((kk & 1) == 0 && (kk >> 1) < kDma && cp.valid) issue_part(cp, kk >> 1, w, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One probability: the lane's score r of token block tb, masked, in log2
// units relative to the row's reference m; tracks the lane's largest score
// and whether any passed m + 64.
__device__ __forceinline__ float tile_prob(const DecodeArgs& a, State& S, const f32x4 (&sacc)[2],
                                           int tok0, int lg, int tb, int r, bool& need) {
  const int t = tok0 + tb * 16 + lg * 4 + r;
  const float v = (t < S.lim) ? sacc[tb][r] * a.scale_log2 : -INFINITY;
  S.tmax = fmaxf(S.tmax, v);
  need |= v > S.m + kRefSlack;
  // (the clamp only matters in a pass that will be redone)
  return (S.m == -INFINITY) ? 0.f : fast_exp2(fminf(v - S.m, kRefSlack));
}

// Online softmax of one tile; lane holds head lr, tokens tb*16 + lg*4 + r.
// Returns the probabilities packed as the B operand (bf16) and adds their
// rounded values to the lane's sum.
//   * The chunk's first tile (first): a row's first scores set its
//     reference, formed across the row's four lanes; a jump past the
//     reference + 64 marks the workgroup for a second pass.
//   * Later tiles: every row with a visible key in the chunk has its
//     reference (the first tile holds the chunk's first key, and visibility
//     is a prefix), so d = s - m is one FMA per score, the jump test is one
//     compare per tile and masking is needed only on a tile that crosses
//     some row's limit.  A row with no reference has no visible key: its
//     d is -inf (m taken as +inf).
__device__ __forceinline__ u16x8 tile_softmax(const DecodeArgs& a, State& S,
                                              const f32x4 (&sacc)[2], int tok0, int lane,
                                              bool first) {
  const int lg = lane >> 4;
  uint32_t pk[4];
  float psum = 0.f;
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  if (first) {
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + tb * 16 + lg * 4 + r;
        mx = fmaxf(mx, (t < S.lim) ? sacc[tb][r] * a.scale_log2 : -INFINITY);
      }
    if (__ballot(mx > S.m + kRefSlack)) {
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      float mass = S.l;
      mass = wave_sum_xor(mass, 16);
      mass = wave_sum_xor(mass, 32);
      if (mx > S.m + kRefSlack && mass == 0.f) S.m = mx;
    }
    bool need = false;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = tile_prob(a, S, sacc, tok0, lg, tb, r, need);
        const float p1 = tile_prob(a, S, sacc, tok0, lg, tb, r + 1, need);
        pk[tb * 2 + r / 2] = pack_bf16x2(p0, p1);
      }
    S.redo |= need;
  } else {
    const float m_eff = S.m == -INFINITY ? INFINITY : S.m;
    float d[2][4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) d[tb][r] = fmaf(sacc[tb][r], a.scale_log2, -m_eff);
    if (__ballot(tok0 + kTile > S.lim)) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tok0 + tb * 16 + lg * 4 + r >= S.lim) d[tb][r] = -INFINITY;
    }
    const float dmx = fmaxf(fmaxf(fmaxf(d[0][0], d[0][1]), fmaxf(d[0][2], d[0][3])),
                            fmaxf(fmaxf(d[1][0], d[1][1]), fmaxf(d[1][2], d[1][3])));
    // (a row without reference gives -inf + inf = NaN, which fmaxf ignores)
    S.tmax = fmaxf(S.tmax, dmx + m_eff);
    S.redo |= dmx > kRefSlack;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; r += 2)
        pk[tb * 2 + r / 2] = pack_bf16x2(fast_exp2(fminf(d[tb][r], kRefSlack)),
                                         fast_exp2(fminf(d[tb][r + 1], kRefSlack)));
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[c]), one2, psum, false);
  S.l += psum;
  return __builtin_bit_cast(u16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
}

// ---- O^T[d, h] += C^T[d, t] P^T[t, h] for the pair's two row blocks and
// this wave's 16 column blocks of tile stage st, probabilities from buffer
// par.  Also issues the copy parts of a later tile (cp).
__device__ __forceinline__ void tile_pv(State& S, int st, int par, int lane, LaneOff lo,
                                        const TileCopy& cp, int w) {
  static_assert(3 * (kDma - 1) < DBH, "a tile's copies fit in the PV steps");
  const int pr = w >> 1, half = w & 1;
  // the wave's columns start at chunk group half * 2 of each latent row
  const MLA_LDS uint8_t* lat = stage_base(st) + half * 512;
  const MLA_LDS uint8_t* pb = (const MLA_LDS uint8_t*)s_p + par * P_BUF + pr * 2 * 256;
  asm volatile("" : "+v"(lo.pv), "+v"(lo.p));
  const u16x8 p0 = *(const MLA_LDS u16x8*)(pb + lo.p);
  const u16x8 p1 = *(const MLA_LDS u16x8*)(pb + lo.p + 256);
  // transpose read: lane (lg, lr) addresses token row lg*4 + lr/4 (and +16),
  // latent dims db*16 + (lr&3)*4 .. +3, i.e. chunk 2db + (lr&3)/2, which sits
  // at ((2(db & 7) + (lr&3)/2) ^ key) in chunk group db >> 3
  auto load_c = [&](int db) -> u16x8 {
    const MLA_LDS uint8_t* p = lat + (lo.pv ^ (uint32_t)((db & 7) << 5)) + (db >> 3) * 256;
    const u16x4 lo4 = lds_read_tr16(p);
    const u16x4 hi4 = lds_read_tr16(p + 16 * LAT_ROW);
    return u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  };
#ifdef MLA_PV_AHEAD
  constexpr int PV_AHEAD = MLA_PV_AHEAD;
#else
  constexpr int PV_AHEAD = 2;
#endif
  u16x8 ca[PV_AHEAD];
#pragma unroll
  for (int j = 0; j < PV_AHEAD; ++j) ca[j] = load_c(j);
#pragma unroll
  for (int db = 0; db < DBH; ++db) {
    const u16x8 av = ca[db % PV_AHEAD];
    if (db + PV_AHEAD < DBH) ca[db % PV_AHEAD] = load_c(db + PV_AHEAD);
    S.o[0][db] = mfma_bf16_16x16x32(av, p0, S.o[0][db]);
    S.o[1][db] = mfma_bf16_16x16x32(av, p1, S.o[1][db]);
    if (db % 3 == 0 && db / 3 < kDma && cp.valid) issue_part(cp, db / 3, w, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass over the chunk's tiles [k0, k0 + n).  Iteration i (0 <= i <= n)
// runs the output product of tile i - 1 and the scores of tile i.
template <typename AfterFirst>
__device__ __forceinline__ void run_pass(const DecodeArgs& a, State& S, const Chunk& ch, int k0,
                                         int n, int w, int lane, AfterFirst after_first) {
  constexpr int D = kDma;
  const LaneOff lo = lane_offsets(lane);
  const int32_t* bt_row = a.block_table + (int64_t)ch.b * a.max_pages;
  PageWindow W;
  W.pg0 = uni(k0 * kTile / kPage);
  W.v = page_window_load(bt_row, a.max_pages, W.pg0, lane);
  auto copy_of = [&](int k, int st, bool valid) {
    const int page = valid ? page_lookup(W, bt_row, a.max_pages, k * kTile / kPage, lane) : 0;
    return tile_copy(a, page, ch.len, k, st, valid);
  };
  // tile 0 first (with whatever the caller loads next); tile 1 once it has
  // landed, so that the first wait is not behind it
  issue_tile(copy_of(k0, 0, true), w, lane);
  after_first();
  // tile 0 and the caller's loads have landed; the query registers are
  // marked used here so that the compiler's own wait for them falls at this
  // point (where it is free) and not after the next copies are in flight
  wait_vm<0>();
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(S.q[kk]));
  barrier();
  if (n > 1) issue_tile(copy_of(k0 + 1, 1, true), w, lane);
  const TileCopy none = tile_copy(a, 0, ch.len, 0, 0, false);
  for (int i = 0; i <= n; ++i) {
    if (i > 0) {
      // this wave's copies of tile i are done once at most D newer ones
      // (tile i + 1's) are outstanding; after the barrier every wave's are,
      // the probabilities of tile i - 1 are stored and stage (i - 2) & 3 is
      // free
      if (i + 1 < n) wait_vm<D>();
      else wait_vm<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier();
    }
    // tile i + 2 goes into the stage tile i - 2 used; its copies ride on the
    // output product when there is one, else on the scores
    const TileCopy c = copy_of(k0 + i + 2, (i + 2) & 3, i + 2 < n);
    if (i > 0) tile_pv(S, (i - 1) & 3, (i - 1) & 1, lane, lo, c, w);
    if (i < n) {
      f32x4 sacc[2];
      tile_qk(S, i & 3, lane, lo, i > 0 ? none : c, w, sacc);
      const u16x8 pf = tile_softmax(a, S, sacc, (k0 + i) * kTile, lane, i == 0);
      *(MLA_LDS u16x8*)((MLA_LDS uint8_t*)s_p + (i & 1) * P_BUF + lo.p + w * 256) = pf;
    }
  }
  // every wave is done with the ring and the probabilities once all have
  // passed this barrier
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
}

// The chunk's partial: o~ / l (rounded to bf16, like the output it feeds)
// and its natural-log log-sum-exp.  The row owners publish 1 / l; each wave
// then scales its columns of the pair's rows.
__device__ __forceinline__ void write_partial(const DecodeArgs& a, State& S, int64_t slot,
                                              int w, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  float* s_inv = (float*)((uint8_t*)s_p + P_BUF);
  float lsum = S.l;
  lsum = wave_sum_xor(lsum, 16);
  lsum = wave_sum_xor(lsum, 32);
  const float lse = lsum > 0.f ? (S.m + __log2f(lsum)) * kLn2 : -INFINITY;
  if (lg == 0) {
    const int row = w * 16 + lr;
    s_inv[row] = lsum > 0.f ? 1.0f / lsum : 0.f;
    a.part_lse[slot * kRowsPerWG + row] = lse;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  const int pr = w >> 1, half = w & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (pr * 2 + j) * 16 + lr;
    const float inv = s_inv[row];
    uint16_t* dst =
        (uint16_t*)a.part_o + (slot * kRowsPerWG + row) * D_LAT + half * DBH * 16 + lg * 4;
#pragma unroll
    for (int db = 0; db < DBH; ++db) {
      const f32x4 v = S.o[j][db] * inv;
      *(u32x2*)(dst + db * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;

  const int64_t nt = plan_total_tiles(a.seqlens, a.batch, a.row_groups, lane);
  if (nt == 0) return;
  const int g = plan_chunk_of_block(
      blockIdx.x, plan_chunks_before(a.seqlens, a.batch, a.row_groups, nt, a.num_wg, lane));
  if (g < 0) return;
  Chunk ch;
  if (!plan_find_chunk(a.seqlens, a.batch, a.row_groups, nt, a.num_wg, g, lane, ch)) return;
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

  // query rows of this unit; the (query, head) row of lane (lg, lr) is
  // R = rg*128 + 16w + lr
  const int rows_total = a.q_len * a.n_heads;
  const uint16_t* qlat = (const uint16_t*)a.q_lat;
  const uint16_t* qpe = (const uint16_t*)a.q_pe;
  State S;
  const int R = ch.rg * kRowsPerWG + w * 16 + lr;
  const bool valid = R < rows_total;
  const int jq = valid ? R / a.n_heads : 0;
  const int hq = valid ? R % a.n_heads : 0;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < DBH; ++db) S.o[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  S.m = -INFINITY;
  S.l = 0.f;
  S.lim = valid ? (a.causal ? ch.len - a.q_len + jq + 1 : ch.len) : 0;
  S.tmax = -INFINITY;
  S.redo = false;
  // the query is loaded right after the first tile's copies are issued, so
  // that the first wait covers the two together
  auto load_query = [&]() {
    const int64_t qrow = ((int64_t)ch.b * a.q_len + jq) * a.n_heads + hq;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u16x8 v;
      if (kk < KS_LAT)
        v = *(const u16x8*)(qlat + qrow * D_LAT + kk * 32 + lg * 8);
      else
        v = *(const u16x8*)(qpe + qrow * D_ROPE + (kk - KS_LAT) * 32 + lg * 8);
      S.q[kk] = valid ? v : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };

  run_pass(a, S, ch, k0, n, w, lane, load_query);

  // rare second pass, with the true row maxima as references, when any row
  // of the workgroup saw a score jump (a row's columns are spread over two
  // waves, so all rows start again).  Each wave posts its flag in the
  // probability buffer, which is free once the pass is over.
  int* s_flag = (int*)s_p;
  if (lane == 0) s_flag[w] = S.redo ? 1 : 0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  const bool any_redo = __ballot(lane < kWaves && s_flag[lane & (kWaves - 1)] != 0) != 0;
  if (any_redo) {
    float mx = S.tmax;
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    S.m = mx;
    S.l = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < DBH; ++db) S.o[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (the pass's first barrier follows every wave's read of the flags)
    run_pass(a, S, ch, k0, n, w, lane, [] {});
  }
  write_partial(a, S, slot, w, lane);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_bf16_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
