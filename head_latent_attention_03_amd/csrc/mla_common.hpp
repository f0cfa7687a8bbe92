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
// The split plan, recomputed identically by the decode and combine kernels
// from the device seqlens (no host round trip).
//
// Work unit u = (b, rg): sequence b, row group rg of kRowsPerWG rows of the
// flattened (query token j, head h) space, rows r = j * n_heads + h.  Unit u
// has tiles_u = ceil(L_b / kTile) tiles of cached tokens; NT = sum of tiles_u.
// For a target of G workgroups, unit u is cut into
//     s_u = min(tiles_u, max(1, floor(G * tiles_u / NT)))
// chunks of near-equal tile counts (none if tiles_u = 0); chunk c covers tiles
// [c * tiles_u / s_u, (c + 1) * tiles_u / s_u).  Chunks are numbered in unit
// order (b-major, rg minor); chunk number = workgroup = partial slot.  At most
// G + (number of units) chunks exist.
__host__ __device__ inline int tiles_of(int len) { return (len + kTile - 1) / kTile; }

__host__ __device__ inline int plan_splits(int tiles_u, int64_t nt, int G) {
  if (tiles_u <= 0) return 0;
  const int64_t s = (int64_t)G * tiles_u / nt;
  return s < 1 ? 1 : (s > tiles_u ? tiles_u : (int)s);
}

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


// Total tiles NT over all units (every lane gets the same value).
__device__ inline int64_t plan_total_tiles(const int32_t* seqlens, int batch, int row_groups,
                                           int lane) {
  int part = 0;
  for (int b = lane; b < batch; b += 64) part += tiles_of(seqlens[b]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
  return (int64_t)uni(part) * row_groups;
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

// Chunks of all units of sequences [0, b_end) (the first chunk number of b_end).
__device__ inline int plan_chunks_before(const int32_t* seqlens, int b_end, int row_groups,
                                         int64_t nt, int G, int lane) {
  int part = 0;
  for (int b = lane; b < b_end; b += 64)
    part += plan_splits(tiles_of(seqlens[b]), nt, G) * row_groups;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
  return uni(part);
}

struct Chunk {
  int b, rg, c, splits, tiles, len;
};

// The chunk numbered g; false if g is past the last chunk.
__device__ inline bool plan_find_chunk(const int32_t* seqlens, int batch, int row_groups,
                                       int64_t nt, int G, int g, int lane, Chunk& out) {
  int base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const int cnt = (b < batch) ? plan_splits(tiles_of(seqlens[b]), nt, G) * row_groups : 0;
    int incl = cnt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m, 64);
      if (lane >= m) incl += o;
    }
    const uint64_t hit = __ballot(base + incl > g);
    if (hit) {
      const int f = uni(__builtin_ctzll(hit));
      const int start = base + uni(__shfl(incl - cnt, f, 64));
      out.b = uni(b0 + f);
      out.len = uni(seqlens[out.b]);
      out.tiles = tiles_of(out.len);
      out.splits = plan_splits(out.tiles, nt, G);
      const int off = g - start;
      out.rg = off / out.splits;
      out.c = off % out.splits;
      return true;
    }
    base += uni(__shfl(incl, 63, 64));
  }
  return false;
}

// The chunk a decode workgroup runs (the three functions above in one pass):
// false if there is none.  Up to 64 sequences, one lane each, the lengths are
// read once and the total, the chunk count and the search all come from
// registers; beyond that the general functions run.
__device__ inline bool plan_locate(const int32_t* seqlens, int batch, int row_groups, int G,
                                   int block, int lane, int& g, Chunk& out) {
  if (batch > 64) {
    const int64_t nt = plan_total_tiles(seqlens, batch, row_groups, lane);
    if (nt == 0) return false;
    g = plan_chunk_of_block(block, plan_chunks_before(seqlens, batch, row_groups, nt, G, lane));
    return g >= 0 && plan_find_chunk(seqlens, batch, row_groups, nt, G, g, lane, out);
  }
  const int len = lane < batch ? seqlens[lane] : 0;
  const int tiles = tiles_of(len);
  int part = tiles;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
  const int64_t nt = (int64_t)uni(part) * row_groups;
  if (nt == 0) return false;
  const int splits = plan_splits(tiles, nt, G);
  const int cnt = splits * row_groups;
  int incl = cnt;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, 64);
    if (lane >= m) incl += o;
  }
  g = plan_chunk_of_block(block, uni(__shfl(incl, 63, 64)));
  if (g < 0) return false;
  const uint64_t hit = __ballot(incl > g);
  const int f = uni(__builtin_ctzll(hit));
  out.b = f;
  out.len = uni(__shfl(len, f, 64));
  out.tiles = tiles_of(out.len);
  out.splits = uni(__shfl(splits, f, 64));
  const int off = g - uni(__shfl(incl - cnt, f, 64));
  out.rg = off / out.splits;
  out.c = off % out.splits;
  return true;
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

// 16-byte global -> LDS copy: lane l's 16 bytes land at lds_base + 16 * l
// (lds_base is wave-uniform).  Written as asm so that the compiler's memory
// model does not see it: otherwise any LDS read it cannot prove disjoint from
// the copy's destination gets a wait for every outstanding VMEM operation.
// The copy has no register result; callers wait for it explicitly with
// s_waitcnt vmcnt before a barrier, and no compiler-visible VMEM load of the
// same wave may rely on a vmcnt count made while a copy is outstanding other
// than a conservative one (the compiler under-counts, which over-waits).
__device__ __forceinline__ void dma16(const void* gsrc, const MLA_LDS uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gsrc)
               : "memory", "m0");
}


// The same copy from a wave-uniform base address held in SGPRs plus a 32-bit
// per-lane byte offset (global_load_lds's saddr form: no 64-bit address
// arithmetic per lane).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff,
                                        const MLA_LDS uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  // (readfirstlane returns int: each half goes through uint32_t so that the
  // low half is zero-extended, never sign-extended into the high half)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
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
