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
// with the absorbed query q~ itself stored e4m3 with one power-of-two scale
// 2^Eq per row (q~ . c_t = 2^Eq s_t (q^ . c^_t)), and the chunk's partial (o~
// normalised by its own softmax sum, its natural-log log-sum-exp) for the
// combine pass.
//
// Mapping onto CDNA4 (4 waves, one per SIMD, 512 registers each):
//   * Wave w owns rows 32w .. 32w+31: its e4m3 query [32 x 512] (64 VGPRs),
//     bf16 q_pe [32 x 64] (16 VGPRs) and its output accumulator [32 x 512]
//     f32 (the 256 accumulation registers).
//   * Scores of a tile, in log2 units relative to a per-row reference m:
//       v_t = g_t (2^Eq q^ . c^_t) + [ (scale log2e q_pe) . k^R_t
//                                      + log2 s_t - m ]
//     The latent product is v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3)
//     with the row's 2^Eq as the B block scale; g_t = scale log2e s_t.  The
//     bracket is one accumulator: a 32x32x16 bf16 "bias" MFMA whose A row of
//     token t is (hi(log2 s_t), lo(log2 s_t), 1) and whose B column of a row
//     is (1, 1, -m) (m rounded to bf16; hi + lo carry log2 s_t to ~2^-16),
//     then the four rotary MFMAs on top.  So 2^v_t = s_t 2^(s[t] - m): the
//     token's scale is already inside.  Each lane ends with head l & 31 and
//     tokens 8(i >> 2) + 4(l >> 5) + (i & 3).
//   * Block-scaled probabilities: per row and tile, e = ceil(max_t v_t - 8.75)
//     and P'_t = e4m3(2^v_t / 2^e), so the tile's largest P' lies in
//     (2^7.75, 2^8.75], below e4m3's 448, and no value needs a running
//     rescale: 2^e is the output product's E8M0 block scale, exact.  The sum
//     l adds the e4m3-rounded P'_t 2^e / s_t, so numerator and denominator
//     carry the same rounding.  m is the row's maximum over the chunk's first
//     tile and never moves; only a tile exponent past 100 (scores more than
//     ~100 log2 units above the first tile's, where the f32 accumulator could
//     overflow) sends the workgroup through a second pass with the row's true
//     maximum as m.
//   * O^T += C^T P'^T on v_mfma_scale_f32_32x32x64_f8f6f4 over a pair of
//     tiles (64 tokens: k-block 0 = tile 2p, k-block 1 = tile 2p + 1, each
//     with its own E8M0 scale per row).  In each lane, operand bytes 0-15 lie
//     in k-block 0 and bytes 16-31 in k-block 1 (measured), and the block
//     scale of k-block kb for row n comes from lane n + 32 kb.  So the B
//     operand is the lane's own 16 probabilities of tile 2p, then its 16 of
//     tile 2p + 1, straight from the softmax registers, and the A operand (c^
//     columns) is four ds_read_b64_tr_b8 per lane and MFMA, two from each
//     tile's stage, in the same token order.
//   * Tile i's scores run beside the softmax of tile i - 1 (independent
//     registers, so its VALU work issues while the MFMAs run); after every
//     second tile the output product of the completed pair follows.  A ring
//     of 7 stages [c^ ; k^R ; s] (21 KiB each) keeps four tiles in flight;
//     each wave copies two latent rows per instruction (4), eight rotary
//     rows (1) and eight scales (1) per tile.  Each wave keeps its own table
//     of per-token factors (g_t, 1/s_t and the bias row), rebuilt per tile.
//   * Keys past the sequence (or chunk) end get the bias -3e38 (so P' = 0)
//     and the factor 1/s_t = 0; rows whose causal limit cuts a tile take a
//     masked path for that tile only.
//   * LDS rows are XOR-swizzled on 16-byte chunks for gfx950's LDS (64 banks
//     of 4 bytes; a 16-byte read serves its lanes in four 16-lane cycles; an
//     8-byte transpose read serves lanes 0-31, then 32-63).  Latent chunk c of
//     token t sits at slot (c & 15) ^ key(t) of its 256-byte group, key(t) =
//     4(t & 3) + ((t >> 2) & 3):
//       - scores: a cycle's 16 lanes read one chunk of 16 tokens 4a + r
//         whose a share a parity; (r, a & 3) takes each of its 16 values once;
//       - transpose: a half-wave reads 2 adjacent chunks of the 8 tokens
//         b + {0, 1, 2, 3, 8, 9, 10, 11} (b = 4hh or 16 + 4hh), whose keys
//         share bit 0 and take the other 8 values, so that the chunk bit
//         completes the 16 slots.
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
constexpr int NQK = KS_LAT + 1 + KS_ROPE;     // score MFMAs per tile (13)
constexpr int DB = D_LAT / 32;                // 32-dim output blocks
constexpr int ROPE_OFF = kTile * LAT_ROW;     // 16 KiB
constexpr int SCALE_OFF = ROPE_OFF + kTile * ROPE_ROW;  // 20 KiB
constexpr int STAGE = 21 * 1024;
constexpr int NSTAGE = 7;
constexpr int AHEAD = NSTAGE - 3;             // tiles in flight (4)
constexpr int NW = kRowsPerWG / 32;           // 4 waves
constexpr int kThreads = 64 * NW;
constexpr int kDma = 6;                       // copies per wave and tile
constexpr float kTop = 8.75f;                 // a tile's largest P' <= 2^8.75 < 448
constexpr int kEmax = 100;                    // tile exponents past this are redone
constexpr float kMasked = -3.0e38f;           // the bias of a key past the end
constexpr uint32_t kOneBf16 = 0x3f80u;

// per-token factors of one tile: g_t = scale log2e s_t, 1/s_t, and the bias
// MFMA's A row (hi(log2 s_t), lo(log2 s_t), 1, 0, ..) as bf16
struct Tab {
  float g[kTile];
  float fb[kTile];
  uint32_t bias[kTile][4];
};

__shared__ __attribute__((aligned(1024))) uint8_t s_ring[NSTAGE * STAGE];
__shared__ __attribute__((aligned(16))) Tab s_tab[NW][2];
__shared__ int s_flag[NW];
static_assert(SCALE_OFF + 2 * kTile * 4 <= STAGE, "stage layout");

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(2))) short i16x2;
typedef MLA_LDS Tab LTab;

// 4-byte global -> LDS copy from a wave-uniform base plus a per-lane byte
// offset: lane l's 4 bytes land at lds_base + 4 l (see dma16_s)
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff,
                                       const MLA_LDS uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 nt"
               :
               : "s"(m0), "v"(voff), "s"((const void*)(uintptr_t)bu)
               : "memory", "m0");
}

__device__ __forceinline__ int lat_key(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int rope_key(int t) { return ((t >> 2) & 3) | (((t >> 1) & 1) << 2); }

__device__ __forceinline__ MLA_LDS uint8_t* stage_base(int st) {
  return (MLA_LDS uint8_t*)s_ring + st * STAGE;
}

// Entries pg .. pg + 3 of a block-table row (clamped to its max_pages
// entries) by scalar loads, waited for in place.  The wait counts scalar
// loads only: it neither holds on the vector loads in flight nor leaves the
// compiler a vector load to wait for, whose wait would count every older
// vector load and copy (so that the prologue's copies would go out one tile
// at a time).  glc reads from L2, past the scalar cache, so no line cached
// there before the table was last written can be seen.
__device__ __forceinline__ void scalar_table_entries4(const int32_t* row, int pg, int max_pages,
                                                      int (&out)[4]) {
  const int32_t* p0 = row + min(pg, max_pages - 1);
  const int32_t* p1 = row + min(pg + 1, max_pages - 1);
  const int32_t* p2 = row + min(pg + 2, max_pages - 1);
  const int32_t* p3 = row + min(pg + 3, max_pages - 1);
  int v0, v1, v2, v3;
  asm volatile(
      "s_load_dword %0, %4, 0x0 glc\n\ts_load_dword %1, %5, 0x0 glc\n\t"
      "s_load_dword %2, %6, 0x0 glc\n\ts_load_dword %3, %7, 0x0 glc\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3)
      : "s"(p0), "s"(p1), "s"(p2), "s"(p3)
      : "memory");
  out[0] = v0;
  out[1] = v1;
  out[2] = v2;
  out[3] = v3;
}

// The score MFMAs, written as volatile asm so that each stays in the step it
// is issued in (as pure builtins the compiler sinks them toward their use in
// the next tile's softmax, which keeps all their LDS operands alive across
// the output product).  Consecutive MFMAs of one chain accumulate in place;
// a VALU read of a chain's result must follow mfma_drain() unless a barrier
// lies between them, and every chain's result must be read: the compiler
// takes an asm output as written when the asm issues and would reuse the
// registers of an unread one at once, while the MFMA still runs and writes
// them later.
//   latent: e4m3 x e4m3, A unscaled (E8M0 127 = 2^0), B (the query) scaled by
//   the row's 2^Eq
__device__ __forceinline__ void mfma_lat_first(f32x16& d, const i32x8& a, const i32x8& b,
                                               int qsc) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(d)
               : "v"(a), "v"(b), "v"(127), "v"(qsc));
}
__device__ __forceinline__ void mfma_lat(f32x16& d, const i32x8& a, const i32x8& b, int qsc) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(d)
               : "v"(a), "v"(b), "v"(127), "v"(qsc));
}
//   bias and rotary: bf16
__device__ __forceinline__ void mfma_bf16_first(f32x16& d, const u16x8& a, const u16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_bf16(f32x16& d, const u16x8& a, const u16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// keeps x computed at this point of the program (an empty volatile asm that
// reads it)
template <typename T>
__device__ __forceinline__ void pin(const T& x) {
  asm volatile("" ::"v"(x));
}

// acc += A B with e4m3 operands, B scaled by 2^(sb - 127) per 32-token block,
// the accumulator pinned to the accumulation registers, which hold exactly
// the wave's output; each block is updated by MFMAs only, and mfma_drain()
// covers the MFMA latency before anything else reads or writes them.
__device__ __forceinline__ void mfma_pv(f32x16& acc, const i32x8& a, const i32x8& b, int sb) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc)
               : "v"(a), "v"(b), "v"(127), "v"(sb));
}

__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// The copies of one tile: wave w's latent rows 8w .. 8w+7 (parts 0..3, two
// 512-byte rows each), their rotary rows (part 4) and all 32 scales (part 5).  Latent and rotary rows past the sequence end re-read its last
// token (so the output product never meets stale bytes); the scales of such
// tokens are whatever the page holds and are never used.
struct TileCopy {
  const uint8_t* lat;
  const uint8_t* rope;
  const float* scale;
  int lim, st;     // tile rows past lim re-read row lim (31 for a full tile)
};

__device__ __forceinline__ TileCopy tile_copy(const DecodeArgs& a, int page, int len, int k,
                                              int st) {
  TileCopy c;
  const int tok0 = k * kTile;
  c.lim = uni(min(len - 1 - tok0, kTile - 1));
  const int64_t row0 = (int64_t)page * kPage + (tok0 % kPage);
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
    const int tc = min(t, c.lim);
    const uint32_t off = (uint32_t)(tc * LAT_ROW + (((lane & 31) ^ lat_key(t)) << 4));
    dma16_s(c.lat, off, dst + (w * 8 + 2 * j) * LAT_ROW);
  } else if (j == 4) {
    const int t = w * 8 + (lane >> 3);
    const int tc = min(t, c.lim);
    const uint32_t off = (uint32_t)(tc * ROPE_ROW + (((lane & 7) ^ rope_key(t)) << 4));
    dma16_s(c.rope, off, dst + ROPE_OFF + w * 8 * ROPE_ROW);
  } else {
    // every wave copies the tile's 32 scales (identical bytes to the same
    // place; lanes 32-63 fill the 128 spare bytes after them), so that no
    // lane is masked off
    dma4_s(c.scale, (uint32_t)((lane & 31) << 2), dst + SCALE_OFF);
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
  u16x8 qpe[KS_ROPE];   // bf16 rotary query times scale log2e (B operand)
  u16x8 qb;             // the bias MFMA's B column: (1, 1, -m) on lanes 0-31
  f32x16 o[DB];         // O^T accumulator: lane holds head l & 31, 16 of the
                        // block's 32 latent dims
  int qsc;              // E8M0 code of the row's query scale
  int lim;              // keys visible to the lane's row: t < lim
  float m;              // reference (log2 units, bf16-representable)
  float l;              // per-lane sum
  float tmax;           // largest tile maximum seen (log2 units, absolute)
  bool redo;            // a tile exponent passed kEmax
};

// Per-lane LDS byte offsets from a stage's base:
//   latent scores, k-step ks, half e:  (qk ^ (((4ks & 15) ^ e) << 4)) + 256 (ks >> 2)
//   rotary scores, k-step k:           rp ^ (2k << 4)
//   transpose, block db, tokens +16j:  (pv ^ (2 (db & 7) << 4)) + 256 (db >> 3) + 8192 j
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
  // 2db + dh; the second read of a tile takes the tokens 16 further on (same
  // keys)
  const int r = n >> 1;
  const int tok = (r < 4) ? 4 * hh + r : 8 + 4 * hh + (r - 4);
  o.pv = (uint32_t)(tok * LAT_ROW + ((dh ^ lat_key(tok)) << 4) + 8 * (n & 1));
  return o;
}

__device__ __forceinline__ const MLA_LDS uint8_t* lds_at(uint32_t a) {
  return (const MLA_LDS uint8_t*)(uintptr_t)a;
}

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS void* p) {
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

__device__ __forceinline__ i32x2 tr8(const MLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)p);
}

// the A operand of output block db: its 32 dims x the lane's 16 tokens of
// tile 2p (stage address ba) then the same 16 of tile 2p + 1 (bb), in the
// order of the probability bytes: 4hh + 0..3, 8 + 4hh + 0..3, then 16 further
__device__ __forceinline__ i32x8 load_v(uint32_t ba, uint32_t bb, int db) {
  const uint32_t x = (uint32_t)((2 * (db & 7)) << 4);
  const int o = (db >> 3) * 256;
  const MLA_LDS uint8_t* pa = lds_at(ba ^ x) + o;
  const MLA_LDS uint8_t* pb = lds_at(bb ^ x) + o;
  const i32x2 a = tr8(pa), b = tr8(pa + 16 * LAT_ROW), c = tr8(pb), d = tr8(pb + 16 * LAT_ROW);
  return i32x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The per-token table of the tile in stage st, for this wave: lane l forms
// token (l & 31)'s entry.  Tokens at or past `end` are keys past the sequence or chunk end.
__device__ __forceinline__ void build_table(const DecodeArgs& a, int st, int tok0, int end,
                                            LTab* tab, int lane) {
  const int t = lane & 31;
  const float s = *(const MLA_LDS float*)(stage_base(st) + SCALE_OFF + 4 * t);
  const bool in = tok0 + t < end;
  // (scales of visible tokens are normal positive numbers, a precondition of
  // the call)
  const float h = in ? __log2f(s) : kMasked;
  const uint32_t hb = pack_bf16x2(h, 0.f) & 0xffffu;
  const float hl = in ? h - __uint_as_float(hb << 16) : 0.f;
  const uint32_t w0 = hb | (pack_bf16x2(hl, 0.f) << 16);
  // (both half-waves write the same values to the same places)
  tab->g[t] = in ? s * a.scale_log2 : 0.f;
  tab->fb[t] = in ? __builtin_amdgcn_rcpf(s) : 0.f;
  *(MLA_LDS u32x4*)tab->bias[t] = u32x4{w0, kOneBf16, 0u, 0u};
}

// The softmax of one tile, cut into slices that a score step runs between its
// MFMAs.  Inputs: the tile's score accumulators (sl, sr), its table and first
// token.  Outputs: the e4m3 probabilities pk (tokens 8g + 4hh + 0..3 in byte
// order, g = 0..3) and the E8M0 code of the row's block scale; l and the row
// state are updated in place.
struct Softmax {
  f32x16 sl, sr;
  const LTab* tab;
  f32x4 gv[4], fv[4];
  float v[16];
  float mx;
  float sc;         // 2^e
  int code;
  uint32_t pk[4];

  // first: the chunk's first tile in a pass that sets the reference m from it
  template <int J>
  __device__ __forceinline__ void slice(State& S, int lane, bool first = false) {
    const int hh = lane >> 5;
    if constexpr (J == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) gv[g] = *(const MLA_LDS f32x4*)&tab->g[8 * g + 4 * hh];
    } else if constexpr (J >= 1 && J <= 4) {
      constexpr int g = J - 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[4 * g + r] = fmaf(sl[4 * g + r], gv[g][r], sr[4 * g + r]);
        pin(v[4 * g + r]);
      }
    } else if constexpr (J == 5) {
      // (a tree of three-input maxima)
      const float m0 = fmaxf(fmaxf(v[0], v[1]), v[2]);
      const float m1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
      const float m2 = fmaxf(fmaxf(v[6], v[7]), v[8]);
      const float m3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
      const float m4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
      mx = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), v[15]));
      pin(mx);
    } else if constexpr (J == 6) {
      // the row's tile maximum: the other half-wave holds the row's other 16
      // tokens
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(mx, __uint_as_float(hh ? sw[0] : sw[1]));
      if (first) {
        // the reference: the first tile's maximum rounded to bf16 (0 for a
        // row that sees none of its keys)
        const float mr = mx > 0.5f * kMasked
                             ? __uint_as_float((pack_bf16x2(mx, 0.f) & 0xffffu) << 16)
                             : 0.f;
        S.m = mr;
        S.tmax = mx;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] -= mr;
        mx -= mr;
      } else {
        S.tmax = fmaxf(S.tmax, mx + S.m);
      }
      const float ef = fminf(fmaxf(__builtin_ceilf(mx - kTop), -126.f), 200.f);
      S.redo |= ef > (float)kEmax;
      const int e = min((int)ef, 127);
      code = e + 127;
      sc = __uint_as_float((uint32_t)code << 23);
      pin(code);
      pin(sc);
    } else if constexpr (J >= 7 && J <= 10) {
      constexpr int g = J - 7;
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = fast_exp2(v[4 * g + r]);
      const i16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, x[0], x[1], sc, false);
      const i16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[2], x[3], sc, true);
      pk[g] = __builtin_bit_cast(uint32_t, w);
      pin(pk[g]);
    } else if constexpr (J == 11) {
#pragma unroll
      for (int g = 0; g < 4; ++g) fv[g] = *(const MLA_LDS f32x4*)&tab->fb[8 * g + 4 * hh];
    } else if constexpr (J == 12 || J == 13) {
      // l += P' 2^e / s_t over the lane's tokens (the scaled conversion gives
      // P' 2^e exactly)
      // (four independent partial sums: no long dependent chain)
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 2 * (J - 12); g < 2 * (J - 12) + 2; ++g) {
        const f32x2 b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pk[g], sc, false);
        const f32x2 b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pk[g], sc, true);
        acc[0] = fmaf(b01[0], fv[g][0], acc[0]);
        acc[1] = fmaf(b01[1], fv[g][1], acc[1]);
        acc[2] = fmaf(b23[0], fv[g][2], acc[2]);
        acc[3] = fmaf(b23[1], fv[g][3], acc[3]);
      }
      S.l += (acc[0] + acc[1]) + (acc[2] + acc[3]);
      pin(S.l);
    }
  }

  __device__ __forceinline__ void all(State& S, int lane, bool first) {
    slice<0>(S, lane);
    slice<1>(S, lane);
    slice<2>(S, lane);
    slice<3>(S, lane);
    slice<4>(S, lane);
    slice<5>(S, lane);
    slice<6>(S, lane, first);
    slice<7>(S, lane);
    slice<8>(S, lane);
    slice<9>(S, lane);
    slice<10>(S, lane);
    slice<11>(S, lane);
    slice<12>(S, lane);
    slice<13>(S, lane);
  }
};

// Rows whose causal limit falls in the tile (starting at tok0): their keys at
// or past the limit get the score kMasked through the bias accumulator (a
// uniform branch, taken on such tiles only).
__device__ __forceinline__ void mask_rows(const State& S, f32x16& sr, int tok0, int lane) {
  if (__ballot(tok0 + kTile > S.lim) != 0) {
    mfma_drain();
    // keys t = tok0 + 4hh + 8(i >> 2) + (i & 3)
    const int r = S.lim - tok0 - 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + (i & 3) >= r) sr[i] = kMasked;
  }
}

// The scores of the tile in stage st into (sl, sr): 8 latent MFMAs, the bias
// MFMA and 4 rotary MFMAs, with (SM) the softmax of the previous tile run in
// slices between them and (COPY) the copies of a later tile issued at steps
// 0, 2, .. 10.  Operand reads run two steps ahead of their MFMAs.
struct FirstReads {
  i32x8 k0, k1;
};

// the latent operands of a tile's first two score steps, issued as soon as
// the tile's stage is ready so that their latency overlaps the work before
// the score step
__device__ __forceinline__ FirstReads first_reads(int st, LaneOff lo) {
  const uint32_t bq = lds_addr(stage_base(st)) + lo.qk;
  return FirstReads{load_k(bq, 0), load_k(bq, 1)};
}

template <bool SM, bool COPY>
__device__ __forceinline__ void score_step(State& S, int st, const LTab* tab, f32x16& sl,
                                           f32x16& sr, Softmax& prev, int lane, LaneOff lo,
                                           const TileCopy& cp, int w, const FirstReads& fr) {
  const uint32_t bq = lds_addr(stage_base(st)) + lo.qk;
  const uint32_t br = lds_addr(stage_base(st)) + lo.rp;
  i32x8 ka0 = fr.k0, ka1 = fr.k1;
  u16x8 ra0, ra1, bias;
#pragma unroll
  for (int j = 0; j < NQK; ++j) {
    if (COPY && j % 2 == 0 && j / 2 < kDma) issue_part(cp, j / 2, w, lane);
    if (j < KS_LAT) {
      const i32x8 cur = (j & 1) ? ka1 : ka0;
      if (j + 2 < KS_LAT) {
        if (j & 1) ka1 = load_k(bq, j + 2);
        else ka0 = load_k(bq, j + 2);
      } else if (j + 2 == KS_LAT) {
        bias = *(const MLA_LDS u16x8*)tab->bias[lane & 31];
      } else {
        ra0 = load_r(br, 0);
      }
      if (j == 0) mfma_lat_first(sl, cur, S.q8[j], S.qsc);
      else mfma_lat(sl, cur, S.q8[j], S.qsc);
    } else if (j == KS_LAT) {
      ra1 = load_r(br, 1);
      mfma_bf16_first(sr, bias, S.qb);
    } else {
      const int k = j - KS_LAT - 1;
      const u16x8 cur = (k & 1) ? ra1 : ra0;
      if (k + 2 < KS_ROPE) {
        if (k & 1) ra1 = load_r(br, k + 2);
        else ra0 = load_r(br, k + 2);
      }
      mfma_bf16(sr, cur, S.qpe[k]);
    }
    if constexpr (SM) {
      switch (j) {
        case 0: prev.template slice<0>(S, lane); break;
        case 1: prev.template slice<1>(S, lane); break;
        case 2: prev.template slice<2>(S, lane); break;
        case 3: prev.template slice<3>(S, lane); break;
        case 4: prev.template slice<4>(S, lane); break;
        case 5: prev.template slice<5>(S, lane); break;
        case 6: prev.template slice<6>(S, lane); break;
        case 7: prev.template slice<7>(S, lane); break;
        case 8: prev.template slice<8>(S, lane); break;
        case 9: prev.template slice<9>(S, lane); break;
        case 10: prev.template slice<10>(S, lane); break;
        case 11: prev.template slice<11>(S, lane); break;
        case 12:
          prev.template slice<12>(S, lane);
          prev.template slice<13>(S, lane);
          break;
        default: break;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The output product of a pair: the lane's probabilities of tile 2p (pa,
// block code ca) and of tile 2p + 1 (pb, cb) times the c^ columns of stages
// sa and sb.
__device__ __forceinline__ void pv_step(State& S, const uint32_t (&pa)[4], int ca,
                                        const uint32_t (&pb)[4], int cb, int sa, int sb, int lane,
                                        LaneOff lo) {
  const i32x8 b = i32x8{(int)pa[0], (int)pa[1], (int)pa[2], (int)pa[3],
                        (int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3]};
  // (the block scale of k-block kb comes from lanes 32 kb ..)
  const int code = (lane >> 5) ? cb : ca;
  const uint32_t ba = lds_addr(stage_base(sa)) + lo.pv;
  const uint32_t bb = lds_addr(stage_base(sb)) + lo.pv;
  i32x8 va0 = load_v(ba, bb, 0), va1 = load_v(ba, bb, 1);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const i32x8 cur = (db & 1) ? va1 : va0;
    if (db + 2 < DB) {
      if (db & 1) va1 = load_v(ba, bb, db + 2);
      else va0 = load_v(ba, bb, db + 2);
    }
    mfma_pv(S.o[db], cur, b, code);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The chunk's one pass over its tiles [k0, k0 + n), as pairs (a last odd
// tile pairs with a phantom tile whose keys all lie past the chunk end).
//   * Prologue: the page window, the query (issued before the window has
//     landed, so that the two latencies overlap) and the copies of tiles 0
//     and 1, all landed before the first barrier (the query registers are
//     marked used there, so that no wait the compiler places for its own
//     loads can fall behind a later copy), then tiles 2 .. AHEAD.  Tile 0's scores and
//     softmax set each row's reference m (first pass); tile 1's scores
//     follow.
//   * Tile i (i >= 1): wait for it (this wave's copies are done once at most
//     AHEAD - 1 newer tiles' are outstanding; after the barrier every wave's
//     are, and every wave is done with the pair before last, whose stages the
//     next copies reuse), copy tile i + AHEAD, build its table, run its
//     scores beside the softmax of tile i - 1 and, for even i, the output
//     product of the pair that softmax completed.  Every tile copies one tile
//     (past the chunk's last tile, a re-read of it into a stage that is not
//     read again), so each wait count is a constant.
template <typename LoadQuery>
__device__ __forceinline__ void run_pass(const DecodeArgs& a, State& S, const Chunk& ch, int k0,
                                         int n, int w, int lane, bool first,
                                         LoadQuery load_query) {
  static_assert(AHEAD + 3 <= NSTAGE, "ring");
  // (a fresh copy of the lane index, so that the per-lane constants below are
  // formed here and not kept alive across the whole pass from the kernel's
  // start, where they would be spilled around the loop)
  asm volatile("" : "+v"(lane));
  const LaneOff lo = lane_offsets(lane);
  const int32_t* bt_row = a.block_table + (int64_t)ch.b * a.max_pages;
  PageWindow W;
  W.pg0 = uni(k0 * kTile / kPage);
  const int k_last = k0 + n - 1;
  const int np = (n + 1) >> 1;
  const int end = min(ch.len, (k0 + n) * kTile);   // keys at or past end are masked
  auto copy_of = [&](int i) {
    const int k = min(k0 + i, k_last);
    const int page = page_lookup(W, bt_row, a.max_pages, k * kTile / kPage, lane);
    return tile_copy(a, page, ch.len, k, i % NSTAGE);
  };
  LTab* tab0 = (LTab*)&s_tab[w][0];
  LTab* tab1 = (LTab*)&s_tab[w][1];
  // the bias B column: (1, 1, -m) for k = 0..2 on lanes 0-31, zero elsewhere
  auto set_qb = [&]() {
    const uint32_t mneg = pack_bf16x2(-S.m, 0.f) & 0xffffu;
    S.qb = (lane >> 5) ? u16x8{}
                       : __builtin_bit_cast(u16x8, u32x4{kOneBf16 | (kOneBf16 << 16), mneg, 0u, 0u});
  };

  // the prologue's tiles 0 .. AHEAD + 1 lie in pages pg0 .. pg0 + 3 (tile i
  // of the chunk is at most (i + 1) / 2 pages past its first)
  static_assert(kPage == 2 * kTile && (AHEAD + 2) / 2 <= 3, "prologue pages");
  if (first) load_query();
  int pgs[4];
  scalar_table_entries4(bt_row, W.pg0, a.max_pages, pgs);
  auto prologue_copy = [&](int i) {
    const int k = min(k0 + i, k_last);
    const int d = uni(k * kTile / kPage - W.pg0);
    const int page = d == 0 ? pgs[0] : (d == 1 ? pgs[1] : (d == 2 ? pgs[2] : pgs[3]));
    return tile_copy(a, page, ch.len, k, i % NSTAGE);
  };
  issue_tile(prologue_copy(0), w, lane);
  issue_tile(prologue_copy(1), w, lane);
  // the page window of the later tiles, landed with the copies
  W.v = page_window_load(bt_row, a.max_pages, W.pg0, lane);
  wait_vm<0>();
  pin(W.v);
  if (first) {
#pragma unroll
    for (int kk = 0; kk < KS_LAT; ++kk) asm volatile("" ::"v"(S.q8[kk]));
#pragma unroll
    for (int kk = 0; kk < KS_ROPE; ++kk) asm volatile("" ::"v"(S.qpe[kk]));
    // (the row scale's exponent field is its E8M0 code)
    S.qsc = (int)((uint32_t)S.qsc >> 23) & 0xff;
    asm volatile("" ::"v"(S.qsc));
    // the softmax scale (log2 units) goes into the rotary query (rounded to
    // bf16 again: 2^-9 relative on the rotary part of a score)
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
    S.m = 0.f;   // until the first tile sets it
  }
  set_qb();
  build_table(a, 0, k0 * kTile, end, tab0, lane);
  barrier();
  const FirstReads fr0 = first_reads(0, lo);
#pragma unroll
  for (int i = 2; i <= AHEAD; ++i) issue_tile(prologue_copy(i), w, lane);

  Softmax sa, sb;   // tiles 2p (its pk, code kept for the pair's product), 2p + 1
  sa.tab = tab0;
  score_step<false, false>(S, 0, tab0, sa.sl, sa.sr, sb, lane, lo, TileCopy{}, w, fr0);
  mask_rows(S, sa.sr, k0 * kTile, lane);
  mfma_drain();
  sa.all(S, lane, first);
  if (first) set_qb();
  {
    wait_vm<(AHEAD - 1) * kDma>();
    barrier();
    const FirstReads fr = first_reads(1, lo);
    const TileCopy c = prologue_copy(1 + AHEAD);
    build_table(a, 1, (k0 + 1) * kTile, end, tab1, lane);
    sb.tab = tab1;
    score_step<false, true>(S, 1, tab1, sb.sl, sb.sr, sa, lane, lo, c, w, fr);
    mask_rows(S, sb.sr, (k0 + 1) * kTile, lane);
  }
  for (int p = 1; p < np; ++p) {
    const int i0 = 2 * p;
    // tile 2p: its scores beside the softmax of tile 2p - 1, then the output
    // product of pair p - 1
    {
      wait_vm<(AHEAD - 1) * kDma>();
      barrier();
      const FirstReads fr = first_reads(i0 % NSTAGE, lo);
      const TileCopy c = copy_of(i0 + AHEAD);
      build_table(a, i0 % NSTAGE, (k0 + i0) * kTile, end, tab0, lane);
      f32x16 nsl, nsr;
      score_step<true, true>(S, i0 % NSTAGE, tab0, nsl, nsr, sb, lane, lo, c, w, fr);
      mask_rows(S, nsr, (k0 + i0) * kTile, lane);
      pv_step(S, sa.pk, sa.code, sb.pk, sb.code, (i0 - 2) % NSTAGE, (i0 - 1) % NSTAGE, lane, lo);
      sa.sl = nsl;
      sa.sr = nsr;
      sa.tab = tab0;
    }
    // tile 2p + 1: its scores beside the softmax of tile 2p
    {
      wait_vm<(AHEAD - 1) * kDma>();
      barrier();
      const FirstReads fr = first_reads((i0 + 1) % NSTAGE, lo);
      const TileCopy c = copy_of(i0 + 1 + AHEAD);
      build_table(a, (i0 + 1) % NSTAGE, (k0 + i0 + 1) * kTile, end, tab1, lane);
      f32x16 nsl, nsr;
      score_step<true, true>(S, (i0 + 1) % NSTAGE, tab1, nsl, nsr, sa, lane, lo, c, w, fr);
      mask_rows(S, nsr, (k0 + i0 + 1) * kTile, lane);
      sb.sl = nsl;
      sb.sr = nsr;
      sb.tab = tab1;
    }
  }
  // the last tile's softmax and the last pair's output product
  mfma_drain();
  sb.all(S, lane, false);
  pv_step(S, sa.pk, sa.code, sb.pk, sb.code, (2 * np - 2) % NSTAGE, (2 * np - 1) % NSTAGE, lane,
          lo);
  // (the last re-reads must land before the stages are reused or the
  // workgroup ends)
  wait_vm<0>();
}

// The chunk's partial: o~ / l (bf16) and its natural-log log-sum-exp, the
// rows staged in the idle ring so that they leave as whole 1 KiB rows.
constexpr int O_PITCH = D_LAT * 2 + 16;
static_assert(NW * 32 * O_PITCH <= NSTAGE * STAGE, "the staged rows fit the ring");

__device__ __forceinline__ void write_partial(const DecodeArgs& a, const State& S, int64_t slot,
                                              int w, int lane) {
  const int lc = lane & 31, hh = lane >> 5;
  mfma_drain();
  const float lsum = wave_sum_xor(S.l, 32);
  const int row = w * 32 + lc;
  if (hh == 0) a.part_lse[slot * kRowsPerWG + row] =
      lsum > 0.f ? (S.m + __log2f(lsum)) * kLn2 : -INFINITY;
  const float f = lsum > 0.f ? 1.0f / lsum : 0.f;
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
  S.m = 0.f;
  S.l = 0.f;
  S.lim = valid ? (a.causal ? ch.len - a.q_len + j + 1 : ch.len) : 0;
  S.tmax = -INFINITY;
  S.redo = false;
  auto load_query = [&]() {
    // (a row past the end reads row 0; its limit 0 masks every key)
    const uint8_t* q8 = (const uint8_t*)a.q_lat + qrow * D_LAT;
    const uint16_t* qpe = (const uint16_t*)a.q_pe + qrow * D_ROPE;
#pragma unroll
    for (int kk = 0; kk < KS_LAT; ++kk) S.q8[kk] = *(const i32x8*)(q8 + kk * 64 + hh * 32);
#pragma unroll
    for (int kk = 0; kk < KS_ROPE; ++kk) S.qpe[kk] = *(const u16x8*)(qpe + kk * 16 + hh * 8);
    // the row scale is a power of two (the absorb pass writes it so); its
    // bits for now, the code once it has landed
    S.qsc = (int)__float_as_uint(a.q_scale[qrow]);
  };

  // the pass, and a rare second one with the true row maxima as references
  // when any tile exponent of the workgroup passed kEmax
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; ++pass) {
    run_pass(a, S, ch, k0, n, w, lane, pass == 0, load_query);
    if (pass == 1) break;
    if (lane == 0) s_flag[w] = S.redo ? 1 : 0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    const bool any_redo = __ballot(lane < NW && s_flag[lane & (NW - 1)] != 0) != 0;
    if (!any_redo) break;
    // (rounded to bf16 like every reference; a row without visible keys
    // keeps m = 0)
    if (S.tmax > 0.5f * kMasked)
      S.m = __uint_as_float((pack_bf16x2(S.tmax, 0.f) & 0xffffu) << 16);
    S.l = 0.f;
    mfma_drain();
#pragma unroll
    for (int db = 0; db < DB; ++db) S.o[db] = f32x16{};
    // (the second pass's first copies go into stages 0 and 1: the barrier
    // above follows every wave's last read of them)
  }
  write_partial(a, S, slot, w, lane);
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s, int grid) {
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
