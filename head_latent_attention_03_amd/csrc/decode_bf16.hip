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
//   * 128 / (16 HB) waves; wave w owns HB 16-row MFMA blocks.  Its absorbed
//     query [16 HB x 576] bf16 stays in VGPRs and its output accumulator
//     [16 HB x 512] f32 in registers for the whole chunk.  HB = 1 (8 waves,
//     two per SIMD) is the default; HB = 2 (4 waves) halves the LDS reads per
//     MFMA but leaves one wave per SIMD to hide every latency alone.
//   * The 32-token tile [c ; k^R] (32 x 1152 B) is brought from HBM straight
//     into LDS with 16-byte global_load_lds (no VGPR staging), through a ring
//     of 4 stages.  The copies of tile i + 3 are issued one per MFMA step of
//     tile i, so that their issue (which stalls while the memory pipeline is
//     full) overlaps the MFMAs; a sequence's page numbers sit one per lane in
//     a VGPR and are read with v_readlane.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows from LDS
//     (ds_read_b128), B = the query from registers.  The accumulator leaves
//     each lane with one head and 8 tokens, which is exactly the B operand of
//     the next product, so the probabilities never touch LDS.
//   * O^T += C^T P^T with the same MFMA: A = C^T read with ds_read_b64_tr_b16
//     (the LDS transpose read), B = P from registers.
//   * The HBM -> LDS copies are issued from inline asm (see dma16_s), so the
//     compiler schedules the LDS reads freely; the ring is guarded by explicit
//     vmcnt waits and one barrier per tile.
//   * Online softmax in fp32 (base 2, scale folded).  Each row keeps a fixed
//     reference maximum, set by its first scores, instead of rescaling the
//     accumulator whenever the maximum grows: probabilities are
//     exp2(s - m_ref) <= 2^64, so nothing overflows, and no cross-lane
//     traffic is needed while scores stay below m_ref + 64.  If a score passes
//     that, the workgroup runs its chunk once more with the true row maxima
//     for the waves that saw it.  The accumulator is thus only ever written by
//     MFMAs.
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
//       - the copies: lat_key(8w + j) = lat_key(8w) ^ 2j, one XOR per row.
//     Rotary chunk c sits at c ^ rope_key(t).
#include "mla_common.hpp"
#include "mla_internal.hpp"

// 16-row MFMA blocks per wave: 1 (8 waves, two per SIMD) or 2 (4 waves)
#ifndef MLA_DECODE_HB
#define MLA_DECODE_HB 1
#endif

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

// Wave geometry: HB 16-row MFMA blocks per wave, 128 / (16 HB) waves.
template <int HB>
struct Geo {
  static constexpr int kWavesWG = kRowsPerWG / (16 * HB);
  static constexpr int kThreads = 64 * kWavesWG;
  static constexpr int kLatRows = kTile / kWavesWG;  // latent rows each wave copies per tile
  static constexpr int kDma = kLatRows + 1;          // copies per wave per tile
};

__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];
__shared__ int s_redo;

// swizzle keys (see the header); both depend on t & 15 only
__device__ __forceinline__ int lat_key(int t) { return ((t & 7) << 1) ^ (((t >> 3) & 1) * 9); }
__device__ __forceinline__ int rope_key(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

// The copies of one tile: this wave's kLatRows latent rows (parts
// 0..kLatRows-1) and the rotary rows of the same tokens (last part, on fewer
// lanes when a wave's rotary rows fill less than 1 KiB).  Tokens past the end
// of the sequence re-read its last token (finite data that the mask then
// ignores), so every wave issues the same count.  The parts are issued one
// per QK k-step of the tile being computed, so their issue (which waits while
// the memory pipeline is full) overlaps the MFMAs.
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

template <int HB>
__device__ __forceinline__ void issue_part(const TileCopy& c, int j, int w, int lane) {
  constexpr int NL = Geo<HB>::kLatRows;
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
    if (NL * ROPE_ROW >= 1024 || lane < NL * 8)
      dma16_s(c.rope, off, dst + LAT_STAGE + w * NL * ROPE_ROW);
  }
}

template <int HB>
__device__ __forceinline__ void issue_tile(const TileCopy& c, int w, int lane) {
#pragma unroll
  for (int j = 0; j < Geo<HB>::kDma; ++j) issue_part<HB>(c, j, w, lane);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int HB>
struct SegState {
  u16x8 q[HB][KS];      // absorbed query (B operand), per 16-row block
  f32x4 o[HB][DB];      // O^T accumulator: lane holds head lr, 4 latent dims
  float m[HB], l[HB];   // reference max (log2 units, scaled) and per-lane sum
  int lim[HB];          // keys visible to the lane's row: t < lim
  float tmax[HB];       // largest score this lane has seen (log2 units, scaled)
  bool redo;            // a score passed m_ref + 64 with mass already accumulated
};

// The chunk's partial: o~ / l (rounded to bf16, like the output it feeds)
// and its natural-log log-sum-exp.
template <int HB>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, SegState<HB>& S,
                                              int64_t slot, int w, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float lsum = S.l[hb];
    lsum = wave_sum_xor(lsum, 16);
    lsum = wave_sum_xor(lsum, 32);
    const float lse = lsum > 0.f ? (S.m[hb] + __log2f(lsum)) * kLn2 : -INFINITY;
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const int row = w * 16 * HB + hb * 16 + lr;
    uint16_t* dst = (uint16_t*)a.part_o + (slot * kRowsPerWG + row) * D_LAT + lg * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 v = S.o[hb][db] * inv;
      *(u32x2*)(dst + db * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (lg == 0) a.part_lse[slot * kRowsPerWG + row] = lse;
  }
}

// Per-lane LDS byte offsets (from a stage's base) of the three read patterns.
// Every address the tile reads is one of them XOR a small constant:
//   QK latent, chunk group v:  qk ^ (v << 6)   ((v*4 + lg) ^ key = (lg ^ key) ^ 4v)
//   QK rotary, chunk group v:  rp ^ (v << 6)
//   PV transpose, column db:   pv ^ ((db & 7) << 5), + 256 per 8 columns
// (the stage base is 1 KiB aligned and the XORed bits never carry).
struct LaneOff {
  uint32_t qk, rp, pv;
};

__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int t1 = lg * 4 + (lr >> 2);
  LaneOff o;
  o.qk = (uint32_t)(lr * LAT_ROW + ((lg ^ lat_key(lr)) << 4));
  o.rp = (uint32_t)(LAT_STAGE + lr * ROPE_ROW + ((lg ^ rope_key(lr)) << 4));
  o.pv = (uint32_t)(t1 * LAT_ROW + ((((lr & 3) >> 1) ^ lat_key(t1)) << 4) + ((lr & 1) << 3));
  return o;
}

// ---- S^T[t, h] = K[t, :] . Q[h, :] for one tile (t = tb*16 + row of the
// 16x16 block).  Also issues the copy parts of a later tile, one per k-step.
template <int HB>
__device__ __forceinline__ void tile_qk(const SegState<HB>& S, int st, int lane, LaneOff lo,
                                        const TileCopy& cp, const TileCopy& cp2, int w,
                                        f32x4 (&sacc)[2][HB]) {
  constexpr int D = Geo<HB>::kDma;
  static_assert(2 * D <= KS, "two tiles' copies fit in the QK k-steps");
  const MLA_LDS uint8_t* lat = stage_base(st);
  asm volatile("" : "+v"(lo.qk), "+v"(lo.rp));
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) sacc[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
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
  constexpr int QK_AHEAD = HB == 1 ? 2 : 3;
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
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      sacc[0][hb] = mfma_bf16_16x16x32(cur0, S.q[hb][kk], sacc[0][hb]);
      sacc[1][hb] = mfma_bf16_16x16x32(cur1, S.q[hb][kk], sacc[1][hb]);
    }
    if (kk < D && cp.valid) issue_part<HB>(cp, kk, w, lane);
    if (kk >= D && kk < 2 * D && cp2.valid) issue_part<HB>(cp2, kk - D, w, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One probability: the lane's score r of token block tb for row block hb,
// masked, in log2 units relative to the row's reference m; tracks the
// lane's largest score and whether any passed m + 64.
template <int HB>
__device__ __forceinline__ float tile_prob(const DecodeArgs& a, SegState<HB>& S,
                                           const f32x4 (&sacc)[2][HB], int tok0, int lg, int hb,
                                           int tb, int r, bool& need) {
  const int t = tok0 + tb * 16 + lg * 4 + r;
  const float v = (t < S.lim[hb]) ? sacc[tb][hb][r] * a.scale_log2 : -INFINITY;
  S.tmax[hb] = fmaxf(S.tmax[hb], v);
  need |= v > S.m[hb] + kRefSlack;
  // (the clamp only matters in a pass that will be redone)
  return (S.m[hb] == -INFINITY) ? 0.f : fast_exp2(fminf(v - S.m[hb], kRefSlack));
}

// Packs the probabilities of row block hb into the PV B operand and adds
// their bf16-rounded values to the lane's sum.
template <int HB>
__device__ __forceinline__ u16x8 tile_pack(SegState<HB>& S, const float (&p)[2][4], int hb) {
  uint32_t pk[4];
  float psum = 0.f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const uint32_t u = pack_bf16x2(p[tb][r], p[tb][r + 1]);
      pk[tb * 2 + r / 2] = u;
      psum += __uint_as_float(u << 16) + __uint_as_float(u & 0xffff0000u);
    }
  S.l[hb] += psum;
  return __builtin_bit_cast(u16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
}

// Online softmax of one tile; lane holds head (hb*16 + lr), tokens
// tb*16 + lg*4 + r.  Common path: every score is below its row's reference
// + 64, so the probabilities follow with no cross-lane traffic.  Otherwise
// (the row's first scores, or a jump) the row maximum is formed across the
// row's four lanes: a row's first scores set its reference, a later jump
// marks the wave for a second pass with the true maxima.
template <int HB>
__device__ __forceinline__ void tile_softmax(const DecodeArgs& a, SegState<HB>& S,
                                             const f32x4 (&sacc)[2][HB], int tok0, int lane,
                                             u16x8 (&pf)[HB]) {
  const int lg = lane >> 4;
  float lmax[HB];
  bool need_lane = false;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + tb * 16 + lg * 4 + r;
        mx = fmaxf(mx, (t < S.lim[hb]) ? sacc[tb][hb][r] * a.scale_log2 : -INFINITY);
      }
    lmax[hb] = mx;
    need_lane |= mx > S.m[hb] + kRefSlack;
  }
  if (__ballot(need_lane)) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float mx = lmax[hb];
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      float mass = S.l[hb];
      mass = wave_sum_xor(mass, 16);
      mass = wave_sum_xor(mass, 32);
      const bool need = mx > S.m[hb] + kRefSlack;
      if (need && mass == 0.f) S.m[hb] = mx;
    }
  }
  bool need = false;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float p[2][4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[tb][r] = tile_prob<HB>(a, S, sacc, tok0, lg, hb, tb, r, need);
    pf[hb] = tile_pack<HB>(S, p, hb);
  }
  S.redo |= need;
}

// ---- O^T[d, h] += C^T[d, t] P^T[t, h] for tile st with probabilities pf.
template <int HB>
__device__ __forceinline__ void tile_pv(SegState<HB>& S, int st, int lane, LaneOff lo,
                                        const u16x8 (&pf)[HB], const TileCopy& cp, int w) {
  constexpr int D = Geo<HB>::kDma;
  static_assert(D <= DB, "a tile's copies fit in the PV steps");
  const MLA_LDS uint8_t* lat = stage_base(st);
  asm volatile("" : "+v"(lo.pv));
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
  constexpr int PV_AHEAD = HB == 1 ? 2 : 4;
#endif
  u16x8 ca[PV_AHEAD];
#pragma unroll
  for (int j = 0; j < PV_AHEAD; ++j) ca[j] = load_c(j);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const u16x8 av = ca[db % PV_AHEAD];
    if (db + PV_AHEAD < DB) ca[db % PV_AHEAD] = load_c(db + PV_AHEAD);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) S.o[hb][db] = mfma_bf16_16x16x32(av, pf[hb], S.o[hb][db]);
    if (db < D && cp.valid) issue_part<HB>(cp, db, w, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass over the chunk's tiles [k0, k0 + n): HBM -> LDS ring of 4 stages
// with three tiles in flight, one barrier per tile; tile i + 3 is copied
// into the stage tile i - 1 used, its copies issued inside QK(i).  Waves with
// active == false only copy their share and keep the barriers.
template <int HB, typename AfterFirst>
__device__ __forceinline__ void run_pass(const DecodeArgs& a, SegState<HB>& S, const Chunk& ch,
                                         int k0, int n, int w, int lane, bool active,
                                         AfterFirst after_first) {
  constexpr int D = Geo<HB>::kDma;
  const LaneOff lo = lane_offsets(lane);
  const int32_t* bt_row = a.block_table + (int64_t)ch.b * a.max_pages;
  PageWindow W;
  W.pg0 = uni(k0 * kTile / kPage);
  W.v = page_window_load(bt_row, a.max_pages, W.pg0, lane);
  auto copy_of = [&](int k, int st, bool valid) {
    const int page = valid ? page_lookup(W, bt_row, a.max_pages, k * kTile / kPage, lane) : 0;
    return tile_copy(a, page, ch.len, k, st, valid);
  };
  // tile 0 first (with whatever the caller loads next); tiles 1 and 2 once
  // it has landed, so that the first wait is not behind them
  issue_tile<HB>(copy_of(k0, 0, true), w, lane);
  after_first();
  // tile 0 and the caller's loads have landed; the query registers are
  // marked used here so that the compiler's own wait for them falls at this
  // point (where it is free) and not after the next copies are in flight
  wait_vm<0>();
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(S.q[hb][kk]));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const TileCopy none = tile_copy(a, 0, ch.len, 0, 0, false);
  for (int i = 0; i < n; ++i) {
    if (i > 0) {
      // this wave's copies of tile i are done once at most
      // D * min(2, n - 1 - i) newer ones are outstanding
      if (i + 2 < n) wait_vm<2 * D>();
      else if (i + 1 < n) wait_vm<D>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // copies issued during this tile, in tile order: tile i + 3 (into the
    // stage tile i - 1 used); during tile 0 also tiles 1 and 2 before it
    TileCopy c0, c1, c2;
    if (i == 0) {
      c0 = copy_of(k0 + 1, 1, n > 1);
      c1 = copy_of(k0 + 2, 2, n > 2);
      c2 = copy_of(k0 + 3, 3, n > 3);
    } else {
      c0 = copy_of(k0 + i + 3, (i + 3) & 3, i + 3 < n);
      c1 = none;
      c2 = none;
    }
    if (active) {
      f32x4 sacc[2][HB];
      u16x8 pf[HB];
      tile_qk<HB>(S, i & 3, lane, lo, c0, c1, w, sacc);
      tile_softmax<HB>(a, S, sacc, (k0 + i) * kTile, lane, pf);
      tile_pv<HB>(S, i & 3, lane, lo, pf, c2, w);
    } else {
      if (c0.valid) issue_tile<HB>(c0, w, lane);
      if (c1.valid) issue_tile<HB>(c1, w, lane);
      if (c2.valid) issue_tile<HB>(c2, w, lane);
    }
  }
  // every wave is done with the ring once all have passed this barrier
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  S.redo = __ballot(S.redo) != 0;
}

template <int HB>
__global__ __launch_bounds__(Geo<HB>::kThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
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
  if (threadIdx.x == 0) s_redo = 0;
  const int k0 = (int)((int64_t)ch.c * ch.tiles / ch.splits);
  const int k1 = (int)((int64_t)(ch.c + 1) * ch.tiles / ch.splits);
  const int n = k1 - k0;
  const int64_t slot = g;

  // query rows of this unit; the (query, head) row of lane (lg, lr) in 16-row
  // block hb is R = rg*128 + 16*HB*w + 16hb + lr
  const int rows_total = a.q_len * a.n_heads;
  const uint16_t* qlat = (const uint16_t*)a.q_lat;
  const uint16_t* qpe = (const uint16_t*)a.q_pe;
  SegState<HB> S;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int R = ch.rg * kRowsPerWG + w * 16 * HB + hb * 16 + lr;
    const bool valid = R < rows_total;
    const int j = valid ? R / a.n_heads : 0;
#pragma unroll
    for (int db = 0; db < DB; ++db) S.o[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    S.m[hb] = -INFINITY;
    S.l[hb] = 0.f;
    S.lim[hb] = valid ? (a.causal ? ch.len - a.q_len + j + 1 : ch.len) : 0;
    S.tmax[hb] = -INFINITY;
  }
  S.redo = false;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // the query is loaded right after the first tile's copies are issued, so
  // that the first wait covers the two together
  auto load_query = [&]() {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int R = ch.rg * kRowsPerWG + w * 16 * HB + hb * 16 + lr;
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
    }
  };

  run_pass<HB>(a, S, ch, k0, n, w, lane, true, load_query);

  // rare second pass, with the true row maxima as references, for the waves
  // that saw a score jump; the whole workgroup keeps the ring going
  if (S.redo && lane == 0) s_redo = 1;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (uni(s_redo)) {
    const bool mine = S.redo;
    if (mine) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float mx = S.tmax[hb];
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        S.m[hb] = mx;
        S.l[hb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) S.o[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    run_pass<HB>(a, S, ch, k0, n, w, lane, mine, [] {});
  }
  write_partial<HB>(a, S, slot, w, lane);
}

constexpr int kHB = MLA_DECODE_HB;

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_bf16_kernel<kHB>, dim3(grid), dim3(Geo<kHB>::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
