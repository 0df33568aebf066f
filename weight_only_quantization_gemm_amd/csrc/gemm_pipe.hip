// W4A16 GEMM for M > 16 activation rows on the fp16 matrix cores.
//
// With more activation rows each weight is reused M times and the product
// turns compute-bound ("AWQ: Activation-aware Weight Quantization for On-Device
// LLM Compression and Acceleration", fdeinterviews.com/papers/awq, paragraph 9:
// under large batches serving becomes more compute-bound).  The codes are
// still dequantized on the fly, never written back as fp16 weights (OpenAlex
// record of the GetMobile AWQ article, abstract).
//
// Design for gfx950 (v_mfma_f32_32x32x16_f16, 160 KB LDS per compute unit):
// the pipeline stage is one 128-channel group.  Both operands of a stage go
// from global memory straight into LDS with global_load_lds_dwordx4 -- the x
// tile [BM][128] fp16 as two 64-channel halves and the packed weight tile
// [128 rows][64 B] -- two or three stages deep, so one or two stages of loads
// are in flight while the matrix cores work.  The block's group scales and
// zeros are copied to LDS once, up front.  A lane's B operand is 8 consecutive channels
// of one weight row, i.e. one packed word: it is unpacked in registers to fp16
// (1024 + code) - (1024 + zero) = code - zero, exactly, and multiplied by the
// group's fp16 scale, which rounds the dequantized weight once to fp16.  The
// matrix core then accumulates all of K in fp32, with no per-group step.
// (Applying the scale in fp32 after each group's MFMAs instead, exact, costs
// 16 more vector instructions per 32 x 32 accumulator tile per group and
// measured 1-3% slower.)
//
// Within a group, the MFMA lanes of half h (l / 32) take channels 64h + 8s ..
// 64h + 8s + 7 at step s = 0..7 in both operands; a lane's 8 B-operand words
// are then contiguous (words 8h .. 8h + 7 of its row).
//
// Blocks: output tile BM x 128 over one or two sets of 4 waves; a set's waves
// sit 2 x 2 (wave tile (BM / 2) x 64) or 1 x 4 (wave tile BM x 32, each
// unpacked weight operand then feeds BM / 32 MFMAs).  Consecutive block ids
// are dispatched to the 8 XCDs in turn,
// so the block order puts the BM-row tiles that share a weight panel on the
// same XCD (block b and b + 8), where they share that XCD's L2.
#include "awq_common.h"
#include "awq_internal.h"
#include "mfma_pipe.h"

#include <type_traits>

namespace awq {

constexpr int kPBN = 128;     // output columns (weight rows) per block
constexpr int kXcds = 8;
constexpr int kLdsBytes = 160 * 1024;

template <int BM, int STAGES, int LDS_BYTES, int KS, int WN_ = 2>
struct PipeShape {
  static constexpr int NW = 4 * KS;                  // waves: KS sets of 4, set i takes channel slice i of a group
  static constexpr int C = kGroup / KS;              // channels of a group per set
  static constexpr int STEPS = C / 16;               // MFMA steps per group per wave
  static constexpr int WN = WN_;                     // a set's 4 waves: 4 / WN along M, WN along N
  static constexpr int WM = 4 / WN;
  static constexpr int TM = BM / WM, TN = kPBN / WN;  // wave tile
  static constexpr int AB = TM / 32;                 // 32-row A blocks per wave
  static constexpr int JB = TN / 32;                 // 32-column B blocks per wave
  static constexpr int A_HALF = BM * 64;             // halfs in one 64-channel half of the x tile
  static constexpr int B_TILE = kPBN * 32;           // halfs in the packed tile (64 B per row)
  static constexpr int STAGE = 2 * A_HALF + B_TILE;  // halfs per stage
  static constexpr int LOADS = 2 * (BM / 8 / NW) + kPBN / 16 / NW;  // direct loads per wave per stage
  static constexpr int PIPE_BYTES = STAGES * STAGE * 2;
  static constexpr int META_BYTES = LDS_BYTES - PIPE_BYTES;  // the block's scales and zeros
  static_assert(META_BYTES > 0 && META_BYTES % 16 == 0, "LDS split");
  static_assert(KS == 1 || KS == 2, "channel split");
  static_assert(KS == 1 || BM * (kPBN + 1) * 4 <= PIPE_BYTES, "set reduction tile must fit the stage buffers");
};

// LDS bytes the block's scales ([128][G] fp16) and zeros ([128][ceil(G/2)]) take.
__host__ __device__ constexpr int64_t pipe_meta_bytes(int64_t G) {
  return ((int64_t)kPBN * G * 2 + 15) / 16 * 16 + (int64_t)kPBN * ((G + 1) / 2);
}

// Copies bytes [0, len) of src (16-byte aligned) to LDS dst (16-byte
// aligned): whole 16-byte chunks straight into LDS by the block's NW waves
// (wave w takes chunks 64(w + NW j) .. +63), the tail bytes (len % 16) by
// plain loads, which are issued first.
template <int NW>
__device__ __forceinline__ void dma_blob(unsigned char* dst, const unsigned char* __restrict__ src, int64_t len,
                                         int wave, int lane, int tid) {
  const int64_t n16 = len / 16;
  if (tid < len - n16 * 16) dst[n16 * 16 + tid] = src[n16 * 16 + tid];
  __asm__ volatile("" ::: "memory");
  wave = __builtin_amdgcn_readfirstlane(wave);
  for (int64_t base = (int64_t)wave * 64; base < n16; base += 64 * NW) {
    const int64_t i = base + lane;
    if (i < n16)
      __builtin_amdgcn_global_load_lds((global_ptr_t)(src + 16 * i), (lds_ptr_t)(dst + 16 * base), 16, 0, 0);
  }
}

// The block's scales ([rows][G] fp16, rows x 2G bytes of the caller's array)
// into LDS in the layout of ScaleSwizzle: with a swizzled layout every row is
// whole 16-byte pieces, and the lane that fills LDS piece v fetches the
// source piece that belongs there.  Otherwise as dma_blob.
template <int NW>
__device__ __forceinline__ void dma_scales(unsigned char* dst, const unsigned char* __restrict__ src, int64_t len,
                                           const ScaleSwizzle& sw, int wave, int lane, int tid) {
  if (sw.mask == 0) {
    dma_blob<NW>(dst, src, len, wave, lane, tid);
    return;
  }
  const int64_t n16 = len / 16;  // a swizzled row is whole pieces
  wave = __builtin_amdgcn_readfirstlane(wave);
  for (int64_t base = (int64_t)wave * 64; base < n16; base += 64 * NW) {
    const int64_t i = base + lane;
    if (i < n16)
      __builtin_amdgcn_global_load_lds((global_ptr_t)(src + 16 * sw.piece_src(i)), (lds_ptr_t)(dst + 16 * base),
                                       16, 0, 0);
  }
}

// KS = 1: one set of 4 waves; MFMA lanes of half h take channels 64h + 8s of
// a group at step s = 0..7.  KS = 2 (two waves per SIMD): 8 waves; waves
// 4i .. 4i + 3 form set i, which covers the whole output tile over channels
// 64i .. 64i + 63 of every group (lane half h: channels 64i + 32h + 8s,
// s = 0..3); the two sets' fp32 partials are summed through LDS at the end,
// in a fixed order.  WN: waves of a set along N (2: 2 x 2, 4: 1 x 4).
// BITS = 3: the packed tile holds each row's 48 bytes of the group (three words
// per 32 channels) back to back, 6 KB of the 8 KB tile, moved as 16-byte pieces
// (the spare lanes of the last instructions copy the last piece into the
// padding, so every wave issues as many loads as at 4 bits); a lane reads the
// three words of its 32-channel chunk and unpacks all 16 channel pairs at once.
// Stream-K work split (Osama, Merrill, Cecka, Garland and Owens, "Stream-K:
// Work-centric Parallel Decomposition for Dense Matrix-Matrix Multiplication
// on the GPU", 2023).  The work is units = tiles x G (one unit: one 128-channel
// group of one output tile); block v of P takes units [v U / P, (v + 1) U / P),
// which may end inside one tile and start inside another.  A block that covers
// a whole tile stores it; otherwise it writes its fp32 partial tile to
// `partials` and counts itself on the tile's counter, and the contributor that
// arrives last adds every contributor's partial in the order of their K
// ranges (so the result does not depend on which one is last), stores the
// tile and resets the counter to 0.  Only a block's first and last tiles can
// be partial: block v keeps them in slots 2 v and 2 v + 1.  With partials ==
// null every block takes one whole tile.
struct StreamK {
  int* counters;    // [tiles]: 0 at entry, left 0
  float* partials;  // [2 P][BM * 128] fp32 in the accumulators' register order; null: whole tiles
  int64_t units;    // tiles * G
  int blocks;       // P, a multiple of 8, at most units
};

// First block (of P) whose unit range holds unit u: the largest v with
// floor(v U / P) <= u.
__host__ __device__ inline int sk_block_of(int64_t u, int64_t U, int P) {
  return (int)(((u + 1) * P + U - 1) / U) - 1;
}

template <int BM, int STAGES, int LDS_BYTES, int KS, int WN, int BITS = 4>
__global__ __launch_bounds__(256 * KS)
__attribute__((amdgpu_waves_per_eu(KS * 163840 / LDS_BYTES, KS * 163840 / LDS_BYTES)))
void gemm_pipe_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed, const f16* __restrict__ scales,
                      const uint8_t* __restrict__ zeros, f16* __restrict__ y, int64_t M, int64_t N, int64_t K, int mt,
                      int nt, StreamK sk) {
  using S = PipeShape<BM, STAGES, LDS_BYTES, KS, WN>;
  constexpr int D = STAGES - 1;  // stages in flight ahead of the one being computed
  __shared__ __attribute__((aligned(16))) f16 lds[LDS_BYTES / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int set = wave >> 2, wq = wave & 3;
  const int wm = wq / WN, wn = wq % WN, h = lane >> 5, l32 = lane & 31;
  const int64_t G = K / kGroup, P2 = (G + 1) / 2;
  const int G32 = (int)G;
  const f16* packed_h = reinterpret_cast<const f16*>(packed);  // a row is K / 4 halfs
  const ScaleSwizzle ssw(G);  // the staged scales' layout

  // This block's units.  Whole tiles: block id -> (m tile, n tile), ids b and
  // b + 8 land on one XCD and share n.  Stream-K: block b runs virtual block
  // v = (b % 8) (P / 8) + b / 8, so an XCD takes one contiguous run of units
  // (tiles t = n_tile mt + m_tile, adjacent tiles sharing a weight panel).
  const int b = (int)blockIdx.x;
  int64_t u0, u1;
  int v = 0;
  if (sk.partials == nullptr) {
    const int chunk = b / (kXcds * mt), rem = b - chunk * kXcds * mt;
    const int nb = chunk * kXcds + rem % kXcds, mb = rem / kXcds;
    if (nb >= nt) return;
    u0 = ((int64_t)nb * mt + mb) * G;
    u1 = u0 + G;
  } else {
    v = (b % kXcds) * (sk.blocks / kXcds) + b / kXcds;
    u0 = (int64_t)v * sk.units / sk.blocks;
    u1 = (int64_t)(v + 1) * sk.units / sk.blocks;
  }

  // fp16x2 (1024, 1024) bit pattern kept in a vector register, so that each
  // channel pair unpacks with one and-or (a VOP3 operand may not be a literal)
  uint32_t magic;
  __asm__ volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  // this lane's channel slice of a group: x half-tile, first 8-channel chunk, first packed word
  const int c0 = set * S::C + h * (S::C / 2);
  const int ahalf = c0 >> 6, achunk = (c0 & 63) >> 3, bchunk = c0 >> 5;

  // D register r of lane l: row 8(r/4) + 4(l/32) + r%4, column l%32 of a 32 x 32 block
  auto store_tile = [&](const f32x16(&acc)[S::AB][S::JB], int64_t m0, int64_t n0) {
#pragma unroll
    for (int a = 0; a < S::AB; ++a)
#pragma unroll
      for (int j = 0; j < S::JB; ++j) {
        const int64_t n = n0 + wn * S::TN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * S::TM + a * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M && n < N) y[m * N + n] = (f16)acc[a][j][r];
        }
      }
  };
  int64_t pend[2];  // tiles this block holds parts of (its first and last)
  int npend = 0;

  for (int64_t u = u0; u < u1;) {
    const int64_t t = u / G;                       // tile of this segment
    const int gl = (int)(u - t * G);               // its groups [gl, gh)
    const int gh = (int)((u1 - t * G) < G ? (u1 - t * G) : G);
    u = t * G + gh;
    const int mb = (int)(t % mt), nb = (int)(t / mt);
    const int64_t m0 = (int64_t)mb * BM, n0 = (int64_t)nb * kPBN;
    const int64_t rows = (N - n0) < kPBN ? (N - n0) : kPBN;  // weight rows of this tile

    lds_barrier();  // the previous segment's LDS (stages, reduction tile) is no longer read
    // Stage slot of group g is (g - gl) % STAGES; past the last group the tail
    // re-reads group gh - 1 into the free slot, so every step issues the same
    // loads and the in-order wait counts below hold on every path.
    TilePlan<BM, S::NW, 64> xplan;
    TilePlan<kPBN, S::NW, 32> wplan;
    xplan.init(x, K, m0, M, wave, lane);
    constexpr int WPER = kPBN / 16 / S::NW;  // packed-tile loads per wave per stage
    const unsigned char* w3src[WPER];
    if constexpr (BITS == 4) {
      wplan.init(packed_h, K / 4, n0, N, wave, lane);
    } else {
      const int wu = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
      for (int jj = 0; jj < WPER; ++jj) {
        int c = (wu * WPER + jj) * 64 + lane;  // 16-byte piece of the tile
        c = c < kPBN * 3 ? c : kPBN * 3 - 1;
        int64_t n = n0 + c / 3;
        n = n < N ? n : N - 1;
        w3src[jj] = reinterpret_cast<const unsigned char*>(packed) + n * (K / 32 * 12) + (c % 3) * 16;
      }
    }
    auto issue = [&](int g, int slot) {
      f16* st = lds + slot * S::STAGE;
      g = g < gh ? g : gh - 1;
      xplan.issue(st, (int64_t)g * kGroup);
      xplan.issue(st + S::A_HALF, (int64_t)g * kGroup + 64);
      if constexpr (BITS == 4) {
        wplan.issue(st + 2 * S::A_HALF, (int64_t)g * 32);
      } else {
        const int wu = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int jj = 0; jj < WPER; ++jj)
          __builtin_amdgcn_global_load_lds((global_ptr_t)(w3src[jj] + (int64_t)g * 48),
                                           (lds_ptr_t)(st + 2 * S::A_HALF + (wu * WPER + jj) * 512), 16, 0, 0);
      }
    };

    // The tile's scales and zeros are two contiguous byte ranges (rows
    // n0 .. n0 + rows - 1 are adjacent); they go to LDS once per segment,
    // ahead of its first stage, so the loop issues no register loads (those
    // would make the in-order vector-memory count unusable for the direct loads).
    unsigned char* meta = reinterpret_cast<unsigned char*>(lds) + S::PIPE_BYTES;
    const int64_t soff = (kPBN * G * 2 + 15) / 16 * 16;
    dma_scales<S::NW>(meta, reinterpret_cast<const unsigned char*>(scales) + n0 * G * 2, rows * G * 2, ssw, wave, lane,
                      tid);
    dma_blob<S::NW>(meta + soff, zeros + n0 * P2, rows * P2, wave, lane, tid);
    const uint16_t* msc = reinterpret_cast<const uint16_t*>(meta);
    const uint8_t* mz = meta + soff;

#pragma unroll
    for (int i = 0; i < D; ++i) issue(gl + i, i);

    int mrow[S::JB], msx[S::JB];  // LDS meta row of the lane's weight rows (clamped to the tile's rows), scale xor
#pragma unroll
    for (int j = 0; j < S::JB; ++j) {
      const int r = wn * S::TN + j * 32 + l32;
      mrow[j] = r < rows ? r : (int)rows - 1;
      msx[j] = ssw.xor_of(mrow[j]);
    }

    f32x16 acc[S::AB][S::JB];
#pragma unroll
    for (int a = 0; a < S::AB; ++a)
#pragma unroll
      for (int j = 0; j < S::JB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][j][r] = 0.f;

    int cur = 0, nxt = D;  // ring slots of stage g and of stage g + D
    for (int g = gl; g < gh; ++g) {
      wait_vmcnt<(D - 1) * S::LOADS>();  // stage g has landed; stages g+1 .. g+D-1 may be pending
      lds_barrier();  // stage g is in LDS for every wave; stage g - 1 is no longer read
      issue(g + D, nxt);
      nxt = nxt + 1 == STAGES ? 0 : nxt + 1;

      const f16* st = lds + cur * S::STAGE;
      cur = cur + 1 == STAGES ? 0 : cur + 1;
      const f16* Ah = st + ahalf * S::A_HALF;
      const f16* Bt = st + 2 * S::A_HALF;
      u32x4 wv[S::JB][S::STEPS / 4];
      ZeroForms zf[S::JB];
      f16x2 sc2[S::JB];
#pragma unroll
      for (int j = 0; j < S::JB; ++j) {
        const int row = wn * S::TN + j * 32 + l32;
#pragma unroll
        for (int q = 0; q < S::STEPS / 4; ++q) {
          if constexpr (BITS == 4) {
            const int sw = (row >> 2) & 3;  // the tile's chunk swizzle (as frag32)
            wv[j][q] = *reinterpret_cast<const u32x4*>(Bt + row * 32 + (((bchunk + q) ^ sw) << 3));
          } else {  // the chunk's three words (row stride 48 bytes)
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(Bt) + row * 12 + (bchunk + q) * 3;
            wv[j][q] = u32x4{wp[0], wp[1], wp[2], 0u};
          }
        }
        zf[j] = zero_forms((mz[mrow[j] * P2 + (g >> 1)] >> (4 * (g & 1))) & 0xFu);
        const uint32_t sbits = msc[mrow[j] * G + (g ^ msx[j])];
        sc2[j] = as_f16x2(sbits | (sbits << 16));
      }
      // Software-pipelined over the MFMA steps of the group: the A fragments
      // and unpacked B operands of step s + 1 are produced while the matrix
      // cores run step s (a scheduling fence closes each step).
      auto unpack = [&](int st_, f16x8(&bq)[S::JB]) {
#pragma unroll
        for (int j = 0; j < S::JB; ++j) {
          if constexpr (BITS == 3) {  // pairs 4 (st_ % 4) .. + 3 of chunk st_ / 4
            const u32x4 w = wv[j][st_ >> 2];
            f16x2 q[4];
#pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
              const int pp = 4 * (st_ & 3) + uu;
              const uint32_t bits =
                  pp < 15 ? ((w[pp / 5] >> (3 * (pp % 5))) & 0x00070007u)
                          : (((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) | ((w[2] >> 13) & 0x00040004u));
              q[uu] = (as_f16x2(bits | magic) - zf[j].zb1) * sc2[j];
            }
            bq[j] = f16x8{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
            continue;
          }
          // exact code - zero, then one rounding by the scale: fp16 of s (q - z)
          const f16x8 sc8 = f16x8{sc2[j].x, sc2[j].y, sc2[j].x, sc2[j].y, sc2[j].x, sc2[j].y, sc2[j].x, sc2[j].y};
          bq[j] = word_minus_zero(wv[j][st_ >> 2][st_ & 3], magic, zf[j]) * sc8;
        }
      };
      f16x8 av[2][S::AB], bq[2][S::JB];
#pragma unroll
      for (int a = 0; a < S::AB; ++a) av[0][a] = frag(Ah, wm * S::TM + a * 32 + l32, achunk);
      unpack(0, bq[0]);
#pragma unroll
      for (int s_ = 0; s_ < S::STEPS; ++s_) {
        const int c = s_ & 1, n = c ^ 1;
        if (s_ + 1 < S::STEPS) {
#pragma unroll
          for (int a = 0; a < S::AB; ++a) av[n][a] = frag(Ah, wm * S::TM + a * 32 + l32, achunk + s_ + 1);
        }
#pragma unroll
        for (int a = 0; a < S::AB; ++a)
#pragma unroll
          for (int j = 0; j < S::JB; ++j)
            acc[a][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[c][a], bq[c][j], acc[a][j], 0, 0, 0);
        if (s_ + 1 < S::STEPS) unpack(s_ + 1, bq[n]);
        __builtin_amdgcn_sched_barrier(0);  // keep each step's work within the step
      }
    }
    wait_vmcnt<0>();  // the tail's redundant LDS loads land before the stage buffers are reused

    if (KS == 2) {  // set 1 hands its partial tile to set 0 through LDS
      float* red = reinterpret_cast<float*>(lds);
      lds_barrier();  // every wave is past its last LDS read of the stage buffers
      if (set == 1) {
#pragma unroll
        for (int a = 0; a < S::AB; ++a)
#pragma unroll
          for (int j = 0; j < S::JB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              red[(wm * S::TM + a * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * (kPBN + 1) + wn * S::TN + j * 32 + l32] =
                  acc[a][j][r];
      }
      lds_barrier();
      if (set == 0) {
#pragma unroll
        for (int a = 0; a < S::AB; ++a)
#pragma unroll
          for (int j = 0; j < S::JB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc[a][j][r] +=
                  red[(wm * S::TM + a * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * (kPBN + 1) + wn * S::TN + j * 32 + l32];
      }
    }

    if (gl == 0 && gh == G32) {  // a whole tile: store it
      if (set == 0) store_tile(acc, m0, n0);
    } else {
      // A part of the tile: its fp32 partial goes to this block's slot for the
      // tile (the tile is the block's first or last), with system-scope
      // stores: the partials are read by blocks on other XCDs, whose L2
      // caches are not coherent with this one's, and such stores go past the
      // L2, so no fence has to write back or invalidate a whole L2.  The
      // block counts itself on the tile after its last segment, when these
      // stores have long completed.
      float* mine = sk.partials + (int64_t)(2 * v + (t == u0 / G ? 0 : 1)) * (BM * kPBN);
      if (set == 0) {
#pragma unroll
        for (int a = 0; a < S::AB; ++a)
#pragma unroll
          for (int j = 0; j < S::JB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              __hip_atomic_store(mine + ((wq * S::AB + a) * S::JB + j) * 1024 + r * 64 + lane, acc[a][j][r],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      pend[npend++] = t;
    }
  }
  if (npend == 0) return;

  // Count this block on the tiles it holds parts of; the contributor that
  // comes last sums all parts in the order of their K ranges and stores the
  // tile.  Contributor c's part of tile t is in slot 2 c when t holds c's
  // first unit, else (t is c's last tile) in slot 2 c + 1.
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed (gfx9: vmcnt counts stores)
  __syncthreads();
  int* flag = reinterpret_cast<int*>(reinterpret_cast<unsigned char*>(lds) + S::PIPE_BYTES);
  if (tid < npend) {
    const int64_t t = pend[tid];
    const int first = sk_block_of(t * G, sk.units, sk.blocks);
    const int count = sk_block_of(t * G + G - 1, sk.units, sk.blocks) - first + 1;
    flag[tid] = __hip_atomic_fetch_add(sk.counters + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == count - 1;
  }
  __syncthreads();
  // The fix-up uses every thread of the block: thread i sums the four
  // consecutive elements 4 (k NT + i) .. + 3 (k < EPT / 4) of the tile's
  // partials, reading two contributors at a time with all their loads in
  // flight.  Plain loads are current here: the parts were stored past the L2
  // (device scope), a kernel starts with no stale L2 lines, and no block of
  // this kernel reads a part's lines before this one.
  constexpr int NT = 256 * KS, EPT = BM * kPBN / NT, V = EPT / 4;
  for (int q = 0; q < npend; ++q) {
    if (!flag[q]) continue;  // block-uniform
    const int64_t t = pend[q];
    const int first = sk_block_of(t * G, sk.units, sk.blocks);
    const int count = sk_block_of(t * G + G - 1, sk.units, sk.blocks) - first + 1;
    auto part = [&](int i) {
      const int c = first + i;
      const int sl = 2 * c + ((int64_t)c * sk.units / sk.blocks >= t * G ? 0 : 1);
      return reinterpret_cast<const f32x4*>(sk.partials + (int64_t)sl * (BM * kPBN)) + tid;
    };
    f32x4 sum[V];
    for (int i = 0; i < count; i += 2) {
      const f32x4* p0 = part(i);
      const f32x4* p1 = part(i + 1 < count ? i + 1 : i);
      f32x4 v0[V], v1[V];
#pragma unroll
      for (int k = 0; k < V; ++k) v0[k] = p0[k * NT];
      if (i + 1 < count) {
#pragma unroll
        for (int k = 0; k < V; ++k) v1[k] = p1[k * NT];
      }
#pragma unroll
      for (int k = 0; k < V; ++k) {
        sum[k] = i == 0 ? v0[k] : sum[k] + v0[k];
        if (i + 1 < count) sum[k] += v1[k];
      }
    }
    // element e of the partial layout: lane e % 64, register r = e / 64 % 16 of
    // accumulator block (wq AB + a) JB + j = e / 1024
    const int64_t m0 = (int64_t)(t % mt) * BM, n0 = (int64_t)(t / mt) * kPBN;
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 4 * (k * NT + tid) + u, el = e & 63, r = (e >> 6) & 15, blk = e >> 10;
        const int j = blk % S::JB, a = (blk / S::JB) % S::AB, w = blk / (S::JB * S::AB);
        const int64_t m = m0 + (w / WN) * S::TM + a * 32 + 8 * (r >> 2) + 4 * (el >> 5) + (r & 3);
        const int64_t n = n0 + (w % WN) * S::TN + j * 32 + (el & 31);
        if (m < M && n < N) y[m * N + n] = (f16)sum[k][u];
      }
    if (tid == 0) __hip_atomic_store(sk.counters + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

constexpr int64_t kCUs = 256;

// Stream-K workspace: 2 P partial tiles of at most 128 x 128 fp32, then one
// int counter per tile (tiles counted at 64 rows, the smaller tile height).
// The counters sit at the same offset for every shape, so a workspace cleared
// once stays valid for calls of any size (each call leaves its counters zero
// and writes partials only below them).
constexpr int64_t kSkPartialBytes = 2 * kCUs * 128 * kPBN * 4;

size_t gemm_pipe_workspace_bytes(int64_t M, int64_t N) {
  return (size_t)(kSkPartialBytes + ((M + 63) / 64 * ((N + kPBN - 1) / kPBN) * 4 + 255) / 256 * 256);
}

static bool pipe_streamk(int64_t M, int64_t N, int64_t G, int64_t BM);

template <int BM, int STAGES, int LDS_BYTES, int KS, int WN, int BITS = 4>
static hipError_t pipe_launch(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                              int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
  const int mt = (int)((M + BM - 1) / BM), nt = (int)((N + kPBN - 1) / kPBN);
  int64_t blocks = (int64_t)((nt + kXcds - 1) / kXcds) * kXcds * mt;
  StreamK sk{nullptr, nullptr, 0, 0};
  const int64_t units = (int64_t)mt * nt * (K / kGroup);
  if (ws != nullptr && pipe_streamk(M, N, K / kGroup, BM)) {
    sk.units = units;
    sk.blocks = (int)(units < kCUs ? units / kXcds * kXcds : kCUs);
    sk.partials = reinterpret_cast<float*>(ws);
    sk.counters = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + kSkPartialBytes);
    blocks = sk.blocks;
  }
  if (KernelPlan* p = active_plan())
    return plan_record(p, "gemm_pipe_kernel<%d,%d,%d,%d,%d,%d> block=%d grid=%lld%s", BM, STAGES, LDS_BYTES, KS, WN,
                       BITS, 256 * KS, (long long)blocks, sk.partials ? " stream-K" : "");
  gemm_pipe_kernel<BM, STAGES, LDS_BYTES, KS, WN, BITS><<<dim3((unsigned)blocks), dim3(256 * KS), 0, st>>>(
      reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed),
      reinterpret_cast<const f16*>(scales), reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), M, N,
      K, mt, nt, sk);
  return hipGetLastError();
}

template <int BM, int STAGES, int LDS_BYTES>
static bool pipe_fits(int64_t G) {
  return pipe_meta_bytes(G) <= PipeShape<BM, STAGES, LDS_BYTES, 1>::META_BYTES;
}

// Measured on the (4096, 11008) and (8192, 28672) layers at M = 128..1024:
// the 1 x 4 wave layout (wave tile 128 x 32: each unpacked weight operand
// feeds four MFMAs) beats 2 x 2 by 10-15 %; two wave sets per block add ~3 %
// at K = 4096 and are neutral at K = 8192.
constexpr int kPipeSets128 = 2, kPipeWN128 = 4;

// Shapes.  64-row x tiles in two channel sets (8 waves) over four stages for
// M <= 64, and for larger M when their rounds over the 256 compute units cost
// less than those of 128-row tiles, a 64-row tile taking ~2/3 of a 128-row
// one.  Measured on the 7B/70B layers: 4096 x 11008 at M = 64 takes 26 us
// against 37 with one set of 4 waves, and at M = 96..128 28 us against 39 with
// 128-row tiles (86 of them: one round either way); 8192 x 8192 at M = 256
// 69 against 79 us (256 tiles of 64 rows against 128 of 128: one round each);
// 8192 x 10240 at M = 256 85 against 111 us the other way (320 tiles of 64
// rows: two rounds), and at M = 512 159 against 174 us (three rounds of 64-row
// tiles against two).  128-row tiles elsewhere (8 waves, two per SIMD, when
// three stages fit); fewer stages where the block's scales and zeros need the
// LDS.

static bool pipe_rows64(int64_t M, int64_t N, int64_t G) {
  if (M <= 64) return true;
  if (!pipe_fits<64, 4, kLdsBytes>(G)) return false;
  const int64_t nt = (N + kPBN - 1) / kPBN;
  const int64_t r64 = ((M + 63) / 64 * nt + kCUs - 1) / kCUs, r128 = ((M + 127) / 128 * nt + kCUs - 1) / kCUs;
  return 2 * r64 < 3 * r128;
}

// Stream-K (with a workspace) where whole tiles leave the compute units
// idle: M > 32, the last round of whole tiles (one block per compute unit)
// fills at most half of the 256 units, and every unit gets at least 8 groups
// (so that the partial tiles' fix-up, a few microseconds, is amortized).
// Measured with the same kernel, whole tiles against stream-K (us): M = 64:
// 8192 x 8192 39.0 (decode ring) against 23.9, 8192 x 10240 48.7 / 32.1,
// 28672 x 8192 116.5 / 66.1, 11008 x 4096 26.9 / 20.2, 4096 x 11008 25.8 /
// 24.9, but 4096 x 4096 (4 groups per unit) 12.9 / 15.1; M = 256: 4096 x
// 4096 25.4 / 20.7, 11008 x 4096 52.8 / 40.0, 28672 x 8192 213 / 144, but
// 4096 x 11008 (172 tiles: 67 % filled) 39.1 / 44.9; full rounds (8192 x 8192
// at M = 256, 4096 x 11008 at M = 1024) within 2 %.  At M <= 32 the decode
// ring kernel was faster on every layer measured.
static bool pipe_streamk(int64_t M, int64_t N, int64_t G, int64_t BM) {
  if (M <= 32) return false;
  const int64_t tiles = (M + BM - 1) / BM * ((N + kPBN - 1) / kPBN);
  const int64_t last = tiles - (tiles - 1) / kCUs * kCUs;  // tiles in the last round
  return 2 * last <= kCUs && tiles * G >= 8 * kCUs;
}

bool gemm_pipe_streamk(int64_t M, int64_t N, int64_t K, int bits) {
  const int64_t G = K / kGroup;
  const bool ok = bits == 3 ? gemm_pipe3_supported(M, N, K) : gemm_pipe_supported(M, N, K);
  return ok && pipe_streamk(M, N, G, pipe_rows64(M, N, G) ? 64 : 128);
}

bool gemm_pipe_supported(int64_t M, int64_t N, int64_t K) {
  const int64_t G = K / kGroup;
  if (!pipe_rows64(M, N, G)) return pipe_fits<128, 2, kLdsBytes>(G);
  return pipe_fits<64, 4, kLdsBytes>(G) || pipe_fits<64, 2, kLdsBytes / 2>(G) || pipe_fits<64, 3, kLdsBytes>(G);
}

hipError_t launch_gemm_pipe(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
  const int64_t G = K / kGroup;
  if (!pipe_rows64(M, N, G)) {
    if (pipe_fits<128, 3, kLdsBytes>(G))
      return pipe_launch<128, 3, kLdsBytes, kPipeSets128, kPipeWN128>(x, packed, scales, zeros, y, M, N, K, ws, st);
    if (pipe_fits<128, 2, kLdsBytes>(G))
      return pipe_launch<128, 2, kLdsBytes, 1, kPipeWN128>(x, packed, scales, zeros, y, M, N, K, ws, st);
    return hipErrorInvalidValue;
  }
  if (pipe_fits<64, 4, kLdsBytes>(G)) return pipe_launch<64, 4, kLdsBytes, 2, 4>(x, packed, scales, zeros, y, M, N, K, ws, st);
  if (pipe_fits<64, 2, kLdsBytes / 2>(G))
    return pipe_launch<64, 2, kLdsBytes / 2, 1, 2>(x, packed, scales, zeros, y, M, N, K, ws, st);
  if (pipe_fits<64, 3, kLdsBytes>(G)) return pipe_launch<64, 3, kLdsBytes, 1, 2>(x, packed, scales, zeros, y, M, N, K, ws, st);
  return hipErrorInvalidValue;
}

// 3-bit codes, M > 16: the same tiles and rules with the 3-bit packed tile.
bool gemm_pipe3_supported(int64_t M, int64_t N, int64_t K) {
  const int64_t G = K / kGroup;
  if (M <= 16) return false;
  if (!pipe_rows64(M, N, G)) return pipe_fits<128, 3, kLdsBytes>(G);
  return pipe_fits<64, 4, kLdsBytes>(G);
}

hipError_t launch_gemm_pipe3(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                             int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
  const int64_t G = K / kGroup;
  if (M <= 16) return hipErrorInvalidValue;
  if (!pipe_rows64(M, N, G)) {
    if (!pipe_fits<128, 3, kLdsBytes>(G)) return hipErrorInvalidValue;
    return pipe_launch<128, 3, kLdsBytes, kPipeSets128, kPipeWN128, 3>(x, packed, scales, zeros, y, M, N, K, ws, st);
  }
  if (!pipe_fits<64, 4, kLdsBytes>(G)) return hipErrorInvalidValue;
  return pipe_launch<64, 4, kLdsBytes, 2, 4, 3>(x, packed, scales, zeros, y, M, N, K, ws, st);
}

}  // namespace awq
