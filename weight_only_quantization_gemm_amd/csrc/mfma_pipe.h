// Building blocks of the pipelined fp16 matrix-core kernels (gfx950): tiles
// of 64 fp16 values per row copied from global memory straight into LDS with
// global_load_lds_dwordx4 (no registers in between, so several pipeline
// stages can be in flight), and conflict-free 16-byte fragment reads.
//
// LDS tile layout: [rows][8 chunks of 16 B]; chunk c of row r sits in slot
// c ^ ((r >> 1) & 7).  A direct load writes 1 KB per wave instruction (lane i
// to bytes 16i..16i+15), i.e. 8 rows; lane i therefore fetches the global
// chunk (i & 7) ^ ((row >> 1) & 7) of row (i >> 3).  A 32x32x16 fragment read
// touches 32 consecutive rows at one logical chunk.  The gfx950 LDS serves a
// 16-byte read for 16 lanes per cycle across 64 four-byte banks (256 B): two
// rows of 128 B per bank line, so the 8 even and the 8 odd rows of any 16
// consecutive rows must each cover the 8 slots; the swizzle period of 16 rows
// does that (measured: 160 B/clk per compute unit, against 120 for a period
// of 8 rows and 32 unswizzled).
#pragma once

#include "awq_common.h"

namespace awq {

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (lgkmcnt and expcnt left at their maxima).
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
  __asm__ volatile("" ::: "memory");
}

typedef void __attribute__((address_space(3))) * lds_ptr_t;
typedef const void __attribute__((address_space(1))) * global_ptr_t;

// Copies rows [row0, row0 + ROWS) x columns [k0, k0 + 64) of a row-major fp16
// matrix (row stride ld elements) into an LDS tile of ROWS x 64, with the
// block's NW waves sharing the ROWS / 8 load instructions.  Rows at or past
// row_end are read from row_end - 1 (valid memory); callers mask them later.
// Issues ROWS / 8 / NW vector-memory operations per wave.
template <int ROWS, int NW>
__device__ __forceinline__ void dl_tile(f16* lds_tile, const f16* __restrict__ g, int64_t ld, int64_t row0,
                                        int64_t row_end, int64_t k0, int wave, int lane) {
  static_assert(ROWS % (8 * NW) == 0, "tile rows must split evenly over the waves");
  constexpr int PER_WAVE = ROWS / 8 / NW;
  wave = __builtin_amdgcn_readfirstlane(wave);  // the LDS destination must be wave-uniform
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int blk = wave * PER_WAVE + j;  // 8-row block written by this instruction
    const int row = blk * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    int64_t r = row0 + row;
    r = r < row_end ? r : row_end - 1;
    const f16* src = g + r * ld + k0 + chunk * 8;
    __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)(lds_tile + blk * 8 * 64), 16, 0, 0);
  }
}

// The 16-byte fragment holding logical chunk c of row r of an LDS tile.
__device__ __forceinline__ f16x8 frag(const f16* lds_tile, int r, int c) {
  return *reinterpret_cast<const f16x8*>(lds_tile + r * 64 + ((c ^ ((r >> 1) & 7)) << 3));
}

// Narrow tiles: 32 fp16 values (4 chunks) per row.  One direct load covers 16
// rows; chunk c of row r sits in slot c ^ ((r >> 2) & 3): four 64-byte rows
// share a 256-byte bank line, so each residue of r mod 4 among 16 consecutive
// rows must cover the 4 slots (measured: 150 B/clk per compute unit, against
// 117 for c ^ ((r >> 1) & 3)).
template <int ROWS, int NW>
__device__ __forceinline__ void dl_tile32(f16* lds_tile, const f16* __restrict__ g, int64_t ld, int64_t row0,
                                          int64_t row_end, int64_t k0, int wave, int lane) {
  static_assert(ROWS % (16 * NW) == 0, "tile rows must split evenly over the waves");
  constexpr int PER_WAVE = ROWS / 16 / NW;
  wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int blk = wave * PER_WAVE + j;  // 16-row block written by this instruction
    const int row = blk * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    int64_t r = row0 + row;
    r = r < row_end ? r : row_end - 1;
    const f16* src = g + r * ld + k0 + chunk * 8;
    __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)(lds_tile + blk * 16 * 32), 16, 0, 0);
  }
}

__device__ __forceinline__ f16x8 frag32(const f16* lds_tile, int r, int c) {
  return *reinterpret_cast<const f16x8*>(lds_tile + r * 32 + ((c ^ ((r >> 2) & 3)) << 3));
}

// The same copies with the per-lane source addresses computed once: a tile
// that moves along k by a uniform offset each stage costs one 64-bit add per
// load instruction.  WIDTH is 64 (layout of dl_tile) or 32 (dl_tile32).
template <int ROWS, int NW, int WIDTH>
struct TilePlan {
  static_assert(WIDTH == 64 || WIDTH == 32 || WIDTH == 16, "tile width");
  static constexpr int ROWS_PER_LOAD = 512 / WIDTH;
  static constexpr int PER_WAVE = ROWS / ROWS_PER_LOAD / NW;
  static_assert(ROWS % (ROWS_PER_LOAD * NW) == 0, "tile rows must split evenly over the waves");
  const f16* src[PER_WAVE];
  int lds_off;  // halfs from the tile start to this wave's first load

  __device__ __forceinline__ void init(const f16* __restrict__ g, int64_t ld, int64_t row0, int64_t row_end, int wave,
                                       int lane) {
    wave = __builtin_amdgcn_readfirstlane(wave);
    lds_off = wave * PER_WAVE * ROWS_PER_LOAD * WIDTH;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave * PER_WAVE + j;
      int row, chunk;
      if (WIDTH == 64) {
        row = blk * 8 + (lane >> 3);
        chunk = (lane & 7) ^ ((row >> 1) & 7);
      } else if (WIDTH == 32) {
        row = blk * 16 + (lane >> 2);
        chunk = (lane & 3) ^ ((row >> 2) & 3);
      } else {
        row = blk * 32 + (lane >> 1);
        chunk = (lane & 1) ^ ((row >> 3) & 1);
      }
      int64_t r = row0 + row;
      r = r < row_end ? r : row_end - 1;
      src[j] = g + r * ld + chunk * 8;
    }
  }

  // Columns [k0, k0 + WIDTH) of the planned rows into lds_tile.
  __device__ __forceinline__ void issue(f16* lds_tile, int64_t k0) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j)
      __builtin_amdgcn_global_load_lds((global_ptr_t)(src[j] + k0),
                                       (lds_ptr_t)(lds_tile + lds_off + j * ROWS_PER_LOAD * WIDTH), 16, 0, 0);
  }
};

// 16-wide tiles (2 chunks of 16 B per row): eight 32-byte rows share a
// 256-byte bank line, so chunk c of row r sits in slot c ^ ((r >> 3) & 1).
__device__ __forceinline__ f16x8 frag16(const f16* lds_tile, int r, int c) {
  return *reinterpret_cast<const f16x8*>(lds_tile + r * 16 + ((c ^ ((r >> 3) & 1)) << 3));
}

// Layout of a block's group scales staged in LDS as [rows][G] fp16.  The
// matrix-core kernels read one scale per row at a fixed group g, from 16 or
// 32 consecutive rows at once; with rows of 2G bytes in a power-of-two
// multiple of 16 bytes those reads pile onto a few of the 64 four-byte banks
// (G = 64: every row starts on one of two banks).  Where a row is CH = G / 8
// 16-byte pieces and CH is a power of two, piece c of row r is therefore
// stored in slot c ^ ((r >> shift) & (CH - 1)), shift = log2 of the rows that
// share one 256-byte bank line: 16 consecutive rows then cover 16 distinct
// bank positions at every g.  Other G keep the plain layout (their row pitch
// already spreads the rows, or a row is not a whole number of pieces).
struct ScaleSwizzle {
  int shift = 0, mask = 0, lg_ch = 0;  // mask 0: plain layout; lg_ch = log2(CH)
  __device__ __forceinline__ explicit ScaleSwizzle(int64_t G) {
    const int64_t ch = G / 8;
    if (G % 8 == 0 && ch > 1 && (ch & (ch - 1)) == 0) {
      mask = (int)ch - 1;
      lg_ch = __builtin_ctzll((unsigned long long)ch);
      shift = lg_ch >= 4 ? 0 : 4 - lg_ch;  // rows of 2G = 2^(lg_ch + 4) bytes, 2^shift of them per 256 bytes
    }
  }
  // XOR that maps group g of row r to its staged element: r G + (g ^ xor_of(r))
  __device__ __forceinline__ int xor_of(int r) const { return ((r >> shift) & mask) << 3; }
  // Source 16-byte piece (counted from the blob's first row) of LDS piece v.
  __device__ __forceinline__ int64_t piece_src(int64_t v) const {
    return mask == 0 ? v : (v ^ (((v >> lg_ch) >> shift) & mask));
  }
};

}  // namespace awq
