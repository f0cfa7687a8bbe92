// Shared device/host definitions of the gfx950 MLA decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// ---------------------------------------------------------------------------
// vector types (integer lanes for bf16/fp8 payloads; __bf16 vectors only at the
// MFMA boundary)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;
typedef __attribute__((ext_vector_type(4))) uint16_t u16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Fixed geometry of the bf16/fp8 decode kernels.
constexpr int kTile = 32;          // cached tokens per pipeline stage
constexpr int kRowsPerWG = 128;    // (query token, head) rows per workgroup
constexpr int kWaves = 4;
constexpr int kPage = 64;

// ---------------------------------------------------------------------------
// The split plan, computed by every decode workgroup from the device seqlens
// (no host round trip); the first chunk of each unit records where the
// combine pass finds the unit's partials.
//
// Work unit u = (b, rg): sequence b, row group rg of kRowsPerWG rows of the
// flattened (query token j, head h) space, rows r = j * n_heads + h.  Unit u
// has tiles_u = ceil(L_b / kTile) tiles of cached tokens; NT = sum of tiles_u.
// Chunks are cut to a length C and a budget B of chunks: with G target
// workgroups and U units, the proportional counts
//     p_u = min(tiles_u, max(1, floor(G * tiles_u / NT)))   (0 if tiles_u = 0)
// decide the budget, B = G when they total at most G (every chunk runs in one
// wave of workgroups) and B = G + U otherwise (many short units: two waves);
// then
//     C = min { c : sum_u ceil(tiles_u / c) <= B },   s_u = ceil(tiles_u / C)
// chunks of unit u.  The proportional counts meet that bound with
// c = max_u ceil(tiles_u / p_u), so no chunk is longer than under them.
// Chunk c of unit u covers tiles [c * tiles_u / s_u, (c + 1) * tiles_u / s_u).
// Chunks are numbered in unit order (b-major, rg minor); chunk number =
// workgroup = partial slot.  At most G + U chunks exist.
__host__ __device__ inline int tiles_of(int len) { return (len + kTile - 1) / kTile; }

__host__ __device__ inline int plan_splits(int tiles_u, int64_t nt, int G) {
  if (tiles_u <= 0) return 0;
  const int64_t s = (int64_t)G * tiles_u / nt;
  return s < 1 ? 1 : (s > tiles_u ? tiles_u : (int)s);
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workgroups are dispatched round-robin over the 8 XCDs.  Give consecutive
// logical ids to workgroups of one XCD so neighbouring chunks (e.g. the chunks
// of both row groups of one sequence) share an L2 and run at the same time.
__device__ inline int xcd_logical_id(int block, int nblocks) {
  if (nblocks % 8 != 0) return block;
  return (block % 8) * (nblocks / 8) + block / 8;
}

// ---------------------------------------------------------------------------
__device__ inline float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ inline float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Rotation of one adjacent pair by pos * theta_i, theta_i = base^(-2i/d_rope).
// The angle (up to ~6.5e4 rad) is formed and reduced to [-pi, pi] in fp64, so
// the fp32 sin/cos that follow see a small argument; the rotation runs in
// fp32.  theta is given in fp64.
__device__ __forceinline__ void rope_pair(float x0, float x1, int pos, double theta, float& y0,
                                          float& y1) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double ang = (double)pos * theta;
  const double red = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));
  float s, c;
  sincosf((float)red, &s, &c);
  y0 = x0 * c - x1 * s;
  y1 = x0 * s + x1 * c;
}

__device__ __forceinline__ double rope_theta(int i, int d_rope, float base) {
  return exp2(-2.0 * (double)i / (double)d_rope * log2((double)base));
}


// Wave-wide integer reductions and scan on DPP lane moves (VALU; no LDS round
// trip) and lane reads.  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowShr1 = 0x111;    // lanes at the start of a row of 16 read 0
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

__device__ __forceinline__ int lane_value(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ inline int wave_sum_int(int v) {
  v += dpp_move<kDppQuadSwap1>(v);
  v += dpp_move<kDppQuadSwap2>(v);
  v += dpp_move<kDppRowRor4>(v);
  v += dpp_move<kDppRowRor8>(v);   // every lane: the sum of its row of 16
  return lane_value(v, 0) + lane_value(v, 16) + lane_value(v, 32) + lane_value(v, 48);
}
__device__ inline int wave_max_int(int v) {
  v = max(v, dpp_move<kDppQuadSwap1>(v));
  v = max(v, dpp_move<kDppQuadSwap2>(v));
  v = max(v, dpp_move<kDppRowRor4>(v));
  v = max(v, dpp_move<kDppRowRor8>(v));
  return max(max(lane_value(v, 0), lane_value(v, 16)), max(lane_value(v, 32), lane_value(v, 48)));
}
// Inclusive prefix sum over the lanes.
__device__ inline int wave_incl_scan(int v, int lane) {
  v += dpp_move<kDppRowShr1>(v);
  v += dpp_move<kDppRowShr2>(v);
  v += dpp_move<kDppRowShr4>(v);
  v += dpp_move<kDppRowShr8>(v);   // the scan within each row of 16
  const int r0 = lane_value(v, 15), r1 = lane_value(v, 31), r2 = lane_value(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// The shortest chunk length c in [ceil(NT / B), longest] whose chunk count
// count(c) = sum_u ceil(tiles_u / c) is at most B, by bisection (count falls
// as c grows, and count(longest) <= B holds).
template <typename Count>
__device__ inline int plan_cut_search(int64_t nt, int64_t budget, int longest, Count count) {
  int lo = (int)((nt + budget - 1) / budget), hi = longest;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (count(mid) <= budget)
      hi = mid;
    else
      lo = mid + 1;
  }
  return hi;
}

// The chunk number a decode workgroup runs, given the total chunk count C, or
// -1 for none.  Workgroups are dealt to the 8 XCDs round-robin (block i to
// XCD i % 8), so chunks are handed out to give every XCD the same share,
// ceil(C / 8), consecutive chunk numbers on one XCD.  Needs a grid of at
// least 8 * ceil(C / 8) workgroups.
__device__ inline int plan_chunk_of_block(int block, int C) {
  const int per = (C + 7) / 8;
  const int k = block / 8;
  if (k >= per) return -1;
  const int g = (block % 8) * per + k;
  return g < C ? g : -1;
}

struct Chunk {
  int b, rg, c, splits, tiles, len;
};

// Fills `out` for chunk g of sequence b (whose first chunk is `start`).
__device__ inline void plan_fill_chunk(int b, int len, int cut, int start, int g, Chunk& out) {
  out.b = uni(b);
  out.len = uni(len);
  out.tiles = tiles_of(out.len);
  out.splits = ceil_div(out.tiles, cut);
  const int off = g - start;
  out.rg = off / out.splits;
  out.c = off % out.splits;
}

// The plan with the lengths of up to 64 * NB sequences held in registers
// (sequence 64 i + lane in len[i]): one read of the lengths, then every
// reduction, the bisection and the search run on registers.
template <int NB>
__device__ inline bool plan_locate_regs(const int32_t* seqlens, int batch, int row_groups, int G,
                                        int block, int lane, int& g, Chunk& out) {
  int len[NB];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = 64 * i + lane;
    len[i] = b < batch ? seqlens[b] : 0;
    sum += tiles_of(len[i]);
  }
  const int64_t nt = (int64_t)wave_sum_int(sum) * row_groups;
  if (nt == 0) return false;
  int ptot = 0, longest = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int t = tiles_of(len[i]);
    const int p = plan_splits(t, nt, G);
    ptot += p;
    longest = max(longest, p > 0 ? ceil_div(t, p) : 0);
  }
  const int64_t budget = (int64_t)wave_sum_int(ptot) * row_groups <= G
                             ? (int64_t)G
                             : (int64_t)G + (int64_t)batch * row_groups;
  const int cut = plan_cut_search(nt, budget, wave_max_int(longest), [&](int c) {
    int part = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) part += ceil_div(tiles_of(len[i]), c);
    return (int64_t)wave_sum_int(part) * row_groups;
  });
  int cnt[NB], incl[NB];
  int base = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    cnt[i] = ceil_div(tiles_of(len[i]), cut) * row_groups;
    incl[i] = base + wave_incl_scan(cnt[i], lane);
    base = lane_value(incl[i], 63);
  }
  g = plan_chunk_of_block(block, base);
  if (g < 0) return false;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint64_t hit = __ballot(incl[i] > g);
    if (hit) {
      const int f = uni(__builtin_ctzll(hit));
      plan_fill_chunk(64 * i + f, lane_value(len[i], f), cut,
                      lane_value(incl[i] - cnt[i], f), g, out);
      return true;
    }
  }
  return false;
}

// The same plan for any batch, reading the lengths again for every pass.
__device__ inline bool plan_locate_mem(const int32_t* seqlens, int batch, int row_groups, int G,
                                       int block, int lane, int& g, Chunk& out) {
  int sum = 0;
  for (int b = lane; b < batch; b += 64) sum += tiles_of(seqlens[b]);
  const int64_t nt = (int64_t)wave_sum_int(sum) * row_groups;
  if (nt == 0) return false;
  int ptot = 0, longest = 0;
  for (int b = lane; b < batch; b += 64) {
    const int t = tiles_of(seqlens[b]);
    const int p = plan_splits(t, nt, G);
    ptot += p;
    longest = max(longest, p > 0 ? ceil_div(t, p) : 0);
  }
  const int64_t budget = (int64_t)wave_sum_int(ptot) * row_groups <= G
                             ? (int64_t)G
                             : (int64_t)G + (int64_t)batch * row_groups;
  const int cut = plan_cut_search(nt, budget, wave_max_int(longest), [&](int c) {
    int part = 0;
    for (int b = lane; b < batch; b += 64) part += ceil_div(tiles_of(seqlens[b]), c);
    return (int64_t)wave_sum_int(part) * row_groups;
  });
  int total = 0;
  for (int b = lane; b < batch; b += 64) total += ceil_div(tiles_of(seqlens[b]), cut) * row_groups;
  g = plan_chunk_of_block(block, wave_sum_int(total));
  if (g < 0) return false;
  int base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const int len = b < batch ? seqlens[b] : 0;
    const int cnt = ceil_div(tiles_of(len), cut) * row_groups;
    const int incl = base + wave_incl_scan(cnt, lane);
    const uint64_t hit = __ballot(incl > g);
    if (hit) {
      const int f = uni(__builtin_ctzll(hit));
      plan_fill_chunk(b0 + f, lane_value(len, f), cut, lane_value(incl - cnt, f), g, out);
      return true;
    }
    base = lane_value(incl, 63);
  }
  return false;
}

// The chunk a decode workgroup runs: false if there is none.
__device__ inline bool plan_locate(const int32_t* seqlens, int batch, int row_groups, int G,
                                   int block, int lane, int& g, Chunk& out) {
  if (batch <= 64) return plan_locate_regs<1>(seqlens, batch, row_groups, G, block, lane, g, out);
  if (batch <= 128) return plan_locate_regs<2>(seqlens, batch, row_groups, G, block, lane, g, out);
  if (batch <= 256) return plan_locate_regs<4>(seqlens, batch, row_groups, G, block, lane, g, out);
  return plan_locate_mem(seqlens, batch, row_groups, G, block, lane, g, out);
}

// 2^x with the hardware v_exp_f32 (results below 2^-126 flush to 0, which
// only drops probabilities that small relative to the row's reference)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ inline float bf16_bits_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

__device__ inline f32x4 mfma_bf16_16x16x32(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// LDS transpose read: in each group of 16 lanes, lane n receives column n of
// the 4 x 16 block of 16-bit elements whose row r, columns 4q..4q+3 are
// addressed by lane 4r + q of that group.
__device__ inline u16x4 lds_read_tr16(const MLA_LDS uint8_t* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)p);
  return __builtin_bit_cast(u16x4, v);
}

// 16-byte global -> LDS copy from a wave-uniform base address held in SGPRs
// plus a 32-bit per-lane byte offset (global_load_lds's saddr form: no 64-bit
// address arithmetic per lane): lane l's 16 bytes land at lds_base + 16 * l
// (lds_base is wave-uniform).  Written as asm so that the compiler's memory
// model does not see it: otherwise any LDS read it cannot prove disjoint from
// the copy's destination gets a wait for every outstanding VMEM operation.
// The copy is non-temporal (nt): the decode reads each cache byte once per
// launch, and a hint that the stream need not stay in L2 and the last-level
// cache leaves room there for the weights and partials that the absorb and
// combine of the same step re-read.
// The copy has no register result; callers wait for it explicitly with
// s_waitcnt vmcnt before a barrier, and no compiler-visible VMEM load of the
// same wave may rely on a vmcnt count made while a copy is outstanding other
// than a conservative one (the compiler under-counts, which over-waits).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff,
                                        const MLA_LDS uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  // (readfirstlane returns int: each half goes through uint32_t so that the
  // low half is zero-extended, never sign-extended into the high half)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(m0), "v"(voff), "s"((const void*)(uintptr_t)bu)
               : "memory", "m0");
}

// A window of 64 consecutive entries of one sequence's block table, one per
// lane, so that a tile's physical page is a v_readlane (no memory latency on
// the copy-issue path).  Pages are looked up in increasing order; a lookup
// past the window reloads it (a plain vector load, which waits for the
// wave's outstanding copies: once per 64 pages).
struct PageWindow {
  int v;     // lane l: block_table[b][pg0 + l] (0 past the row)
  int pg0;
};

__device__ inline int page_window_load(const int32_t* bt_row, int max_pages, int pg0, int lane) {
  const int p = pg0 + lane;
  return p < max_pages ? bt_row[p] : 0;
}

__device__ __forceinline__ int page_lookup(PageWindow& W, const int32_t* bt_row, int max_pages,
                                           int pg, int lane) {
  int page;
  if (uni(pg - W.pg0) >= 64) {
    W.pg0 = uni(pg);
    W.v = page_window_load(bt_row, max_pages, W.pg0, lane);
    page = __builtin_amdgcn_readlane(W.v, 0);
  } else {
    page = __builtin_amdgcn_readlane(W.v, uni(pg - W.pg0));
  }
  return page;
}

}  // namespace mla
