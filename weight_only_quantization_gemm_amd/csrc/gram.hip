// G = X^T X of the calibration rows, [K][K], accumulated in fp64 and stored
// rounded to fp32.  It turns the search's output MSE ||X E^T||^2 into
// sum_n E_n G E_n^T, whose cost no longer grows with the number of
// calibration rows.
//
// fp16 x fp16 products are exact in fp32; the matrix cores
// (v_mfma_f32_32x32x16_f16) accumulate 256 rows at a time in fp32 and the
// partial is then added into fp64 registers, so rounding error grows with 256
// rows, not with M.  Only 128 x 128 tiles on or above the diagonal are
// computed; an off-diagonal tile is also written transposed, through LDS.
//
// Pipeline: the calibration rows are consumed 64 at a time; both operand
// tiles (rows of X^T) go straight from global memory into LDS
// (global_load_lds_dwordx4), two stages deep: one stage of loads is in flight
// while the matrix cores work on the other.  At 64 KB of LDS and 246 VGPRs two
// blocks share a compute unit (two waves per SIMD), so one block's fp64 flushes,
// barriers and fragment reads overlap the other's MFMAs.  Measured on 65,536
// rows: K = 4096 1.93 ms (four stages at one block per unit: 2.32 ms), K = 11008
// 10.2 ms (11.6 ms); the kernel before the per-lane load plans and fragment
// double-buffering took 3.7 and 17.8 ms (19 vector instructions per MFMA, most
// of them 64-bit address arithmetic recomputed every stage).
#include "awq_common.h"
#include "awq_internal.h"
#include "mfma_pipe.h"

namespace awq {

constexpr int kGT = 128;          // tile of G
constexpr int kGStages = 2;       // pipeline depth: 64 KB of LDS, two blocks per compute unit
constexpr int kGFlush = 4;        // stages (x 64 rows) per fp32 partial
constexpr int kGLoadsPerWave = 2 * kGT / 8 / 4;  // direct loads per wave per stage (A and B)

// Tile order.  The upper-triangle tiles (I <= J) are grouped into 4 x 4
// super-tiles (SI, SJ), SI <= SJ, numbered row by row; XCD x (block ids b with
// b % 8 == x, which the dispatcher places on XCD x) works through super-tiles
// x, x + 8, x + 16, ..., each one's tiles in turn, so the 32 blocks an XCD
// runs at once read about 8 distinct row panels of X^T and its L2 serves each
// panel chunk to several blocks.
constexpr int kGS = 4;

__host__ __device__ inline int gram_super_tiles(int nb) { return (nb + kGS - 1) / kGS; }

// tiles of super-tile (si, sj) that lie on or above the diagonal
__host__ __device__ inline int gram_super_count(int si, int sj, int nb) {
  const int ni = (nb - kGS * si) < kGS ? (nb - kGS * si) : kGS;
  const int nj = (nb - kGS * sj) < kGS ? (nb - kGS * sj) : kGS;
  return si == sj ? ni * (ni + 1) / 2 : ni * nj;
}

// (I, J) of the q-th tile on XCD x; false past the XCD's last tile
__host__ __device__ inline bool gram_tile(int x, int q, int nb, int& I, int& J) {
  const int ns = gram_super_tiles(nb);
  int si = 0, sj = 0, s = 0;  // super-tile s = (si, sj), row-major over si <= sj
  auto advance = [&](int steps) {
    for (int k = 0; k < steps; ++k) {
      if (++sj == ns) {
        ++si;
        sj = si;
      }
      ++s;
    }
  };
  advance(x);
  const int total = ns * (ns + 1) / 2;
  while (s < total) {
    const int c = gram_super_count(si, sj, nb);
    if (q < c) {
      const int ni = (nb - kGS * si) < kGS ? (nb - kGS * si) : kGS;
      const int nj = (nb - kGS * sj) < kGS ? (nb - kGS * sj) : kGS;
      int i = 0, j = 0;
      if (si == sj) {  // row i holds ni - i tiles (j = i .. ni - 1)
        int r = q;
        while (r >= ni - i) {
          r -= ni - i;
          ++i;
        }
        j = i + r;
      } else {
        i = q / nj;
        j = q - i * nj;
      }
      (void)ni;
      I = kGS * si + i;
      J = kGS * sj + j;
      return true;
    }
    q -= c;
    advance(8);
  }
  return false;
}

// Work plan.  XCD x holds 64 blocks at once (two per compute unit), so its n_x
// tiles take n_x / 64 full rounds and a last round of L_x = n_x % 64 tiles; at
// K = 4096 (528 tiles, 58-74 per XCD) four XCDs had a second round of 4-10
// tiles that took over half as long as the first.  Each of those L_x tiles is
// therefore cut along the
// calibration rows into S_x = 64 / L_x pieces of whole 256-row flush chunks
// (S_x at most the chunk count): the pieces run side by side, each writes its
// fp64 partial tile to a buffer, and a fix-up pass adds every tile's pieces in
// piece order, so the result is deterministic (it can differ from the uncut
// sum in the last bit of fp64, being grouped differently).  Only the XCDs with
// the most rounds are cut, and only if each of their last rounds can be cut at
// least 4 ways (at most 16 tiles); otherwise every tile stays whole:
// measured at K = 11008, where they held 6-30 tiles per XCD, cutting saved
// nothing, since a round that few blocks share runs faster than a full one
// and the XCD with the most tiles sets the time.  At K = 4096 on 65,536 rows
// the Gram takes 1.6 ms cut (fix-up pass 18 us), 2.2-2.5 ms whole.
constexpr int kGramSlots = 64;     // blocks an XCD holds at once
constexpr int kGramMinPieces = 4;  // a last round of more than 16 tiles stays whole
constexpr int kGramStrip = 8;      // tile rows per fix-up block

struct GramPlan {
  int full[8];        // tiles of XCD x run whole (the first full[x] of its list)
  int left[8];        // tiles of XCD x cut into pieces (the next left[x])
  int pieces[8];      // pieces per cut tile on XCD x
  int piece_base[8];  // first partial-buffer slot of XCD x
  int blocks_per_xcd;
  int fixup_per_xcd;
  int piece_slots;    // partial tiles in the buffer
};

__host__ __device__ inline GramPlan gram_plan(int64_t K, int64_t Mp) {
  const int nb = (int)(K / kGT), ns = gram_super_tiles(nb);
  const int chunks = (int)((Mp / 64 + kGFlush - 1) / kGFlush);
  int per[8] = {0, 0, 0, 0, 0, 0, 0, 0}, s = 0;
  for (int si = 0; si < ns; ++si)
    for (int sj = si; sj < ns; ++sj, ++s) per[s % 8] += gram_super_count(si, sj, nb);
  // The XCDs with the most rounds set the time: cut their last rounds, and only
  // if each of them can be cut at least kGramMinPieces ways.
  int L[8], S[8], most = 0;
  for (int x = 0; x < 8; ++x) {
    L[x] = per[x] % kGramSlots;
    S[x] = L[x] > 0 ? kGramSlots / L[x] : 1;
    S[x] = S[x] < chunks ? S[x] : chunks;
    const int rounds = (per[x] + kGramSlots - 1) / kGramSlots;
    most = rounds > most ? rounds : most;
  }
  bool cut = true;
  for (int x = 0; x < 8; ++x)
    if ((per[x] + kGramSlots - 1) / kGramSlots == most) cut = cut && L[x] > 0 && S[x] >= kGramMinPieces;
  GramPlan p{};
  int slots = 0;
  for (int x = 0; x < 8; ++x) {
    const bool c = cut && L[x] > 0 && (per[x] + kGramSlots - 1) / kGramSlots == most;
    p.full[x] = c ? per[x] - L[x] : per[x];
    p.left[x] = c ? L[x] : 0;
    p.pieces[x] = c ? S[x] : 1;
    p.piece_base[x] = slots;
    slots += p.left[x] * p.pieces[x];
    const int blocks = p.full[x] + p.left[x] * p.pieces[x];
    p.blocks_per_xcd = blocks > p.blocks_per_xcd ? blocks : p.blocks_per_xcd;
    p.fixup_per_xcd = p.left[x] > p.fixup_per_xcd ? p.left[x] : p.fixup_per_xcd;
  }
  p.piece_slots = slots;
  return p;
}

// Block q of XCD x: its tile (the XCD's tq-th; -1 for no work), the stages
// [t0, t1) of 64 calibration rows it adds up, and for a piece of a cut tile its
// slot in the partial buffer (-1 for a whole tile).
struct GramWork {
  int tq, slot, t0, t1;
};

__host__ __device__ inline GramWork gram_work(const GramPlan& plan, int x, int q, int64_t Mp) {
  const int stages = (int)(Mp / 64), chunks = (stages + kGFlush - 1) / kGFlush;
  if (q < plan.full[x]) return {q, -1, 0, stages};
  const int u = q - plan.full[x], S = plan.pieces[x];
  if (u >= plan.left[x] * S) return {-1, -1, 0, 0};
  const int piece = u % S;
  const int t0 = (int)((int64_t)piece * chunks / S) * kGFlush;
  const int t1 = (int)((int64_t)(piece + 1) * chunks / S) * kGFlush;
  return {plan.full[x] + u / S, plan.piece_base[x] + u, t0, t1 < stages ? t1 : stages};
}

size_t gram_partial_bytes(int64_t K, int64_t Mp) {
  return (size_t)gram_plan(K, Mp).piece_slots * kGT * kGT * sizeof(double);
}

// Writes the block's fp64 tile (D layout: register r of lane l of wave (wm, wn),
// 2 x 2 blocks of 32 x 32) to G rounded to fp32, and off the diagonal its mirror:
// 64 rows at a time staged in LDS, then written row-coalesced.
__device__ inline void gram_store(const double (&acc64)[2][2][16], int I, int J, int64_t K, float* __restrict__ G,
                                  float* tile, int tid, int wm, int wn, int lane) {
  const int64_t r0 = (int64_t)I * kGT, c0 = (int64_t)J * kGT;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lds_barrier();  // the LDS (or the previous half) is no longer read
    if (wm == h) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = wn * 64 + b * 32 + (lane & 31);
            tile[row * (kGT + 1) + col] = (float)acc64[a][b][r];
          }
    }
    __syncthreads();
    for (int i = tid; i < 64 * kGT; i += 256) {
      const int ry = i >> 7, cx = i & 127;
      G[(r0 + 64 * h + ry) * K + c0 + cx] = tile[ry * (kGT + 1) + cx];
    }
    if (I != J) {
      for (int i = tid; i < 64 * kGT; i += 256) {
        const int cy = i >> 6, rx = i & 63;  // mirrored row c0 + cy, column r0 + 64 h + rx
        G[(c0 + cy) * K + r0 + 64 * h + rx] = tile[rx * (kGT + 1) + cy];
      }
    }
  }
}

// Xt: fp16 [K][Mp] (rows of X^T), Mp % 64 == 0, K % 128 == 0.  Block: 4 waves
// in 2 x 2, each a 64 x 64 tile of 2 x 2 32x32x16 MFMAs; D register r of lane l
// is D[8*(r/4) + 4*(l/32) + r%4][l%32].  STAGES stages of 64 rows go straight
// into LDS; the per-lane source addresses are computed once (a stage costs one
// 64-bit add per load), and past the last stage the tail re-reads it into the
// free slot, so every step waits for the same count of loads and the loop has no
// branch on the pipeline's fill.  With two stages (64 KB of LDS) two blocks share
// a compute unit, two waves per SIMD.
template <int STAGES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(STAGES == 2 ? 2 : 1, STAGES == 2 ? 2 : 1)))
void gram_kernel(const f16* __restrict__ Xt, int64_t Mp, int64_t K, float* __restrict__ G,
                 double* __restrict__ partial, GramPlan plan) {
  constexpr int D = STAGES - 1;  // stages in flight ahead of the one computed
  __shared__ __attribute__((aligned(16))) f16 lds[STAGES][2][kGT * 64];
  const int nb = (int)(K / kGT);
  const GramWork wk = gram_work(plan, (int)(blockIdx.x & 7), (int)(blockIdx.x >> 3), Mp);
  int I, J;
  if (wk.tq < 0 || !gram_tile((int)(blockIdx.x & 7), wk.tq, nb, I, J)) return;
  const int slot = wk.slot, t0 = wk.t0, T = wk.t1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)I * kGT, c0 = (int64_t)J * kGT;

  TilePlan<kGT, 4, 64> pa, pb;
  pa.init(Xt, Mp, r0, K, wave, lane);
  pb.init(Xt, Mp, c0, K, wave, lane);
  auto issue = [&](int t, int ring) {
    const int64_t k0 = (int64_t)(t < T ? t : T - 1) * 64;
    pa.issue(lds[ring][0], k0);
    pb.issue(lds[ring][1], k0);
  };

  f32x16 acc[2][2];
  double acc64[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[a][b][r] = 0.f;
        acc64[a][b][r] = 0.0;
      }

  for (int t = 0; t < D; ++t) issue(t0 + t, t);
  int cur = 0, nxt = D;  // ring slots of stage t and of stage t + D
  for (int t = t0; t < T; ++t) {
    wait_vmcnt<(D - 1) * kGLoadsPerWave>();  // stage t has landed; later ones may be pending
    lds_barrier();  // every wave's part of stage t is in LDS; stage t - 1 is no longer read
    issue(t + D, nxt);
    nxt = nxt + 1 == STAGES ? 0 : nxt + 1;
    const f16* A = lds[cur][0];
    const f16* B = lds[cur][1];
    cur = cur + 1 == STAGES ? 0 : cur + 1;
    // Fragments of step s + 1 are read while the matrix cores run step s.
    f16x8 av[2][2], bv[2][2];
    auto load = [&](int s, int buf) {
      const int c = 2 * s + (lane >> 5);
#pragma unroll
      for (int a = 0; a < 2; ++a) av[buf][a] = frag(A, wm * 64 + a * 32 + (lane & 31), c);
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[buf][b] = frag(B, wn * 64 + b * 32 + (lane & 31), c);
    };
    load(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) load(s + 1, (s + 1) & 1);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s & 1][a], bv[s & 1][b], acc[a][b], 0, 0, 0);
    }
    if ((t + 1) % kGFlush == 0 || t + 1 == T) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc64[a][b][r] += (double)acc[a][b][r];
            acc[a][b][r] = 0.f;
          }
    }
  }
  wait_vmcnt<0>();  // the tail's redundant loads land before the buffers are reused

  static_assert(STAGES * 2 * kGT * 64 * 2 >= 64 * (kGT + 1) * 4, "the fp32 half tile must fit the stage buffers");
  if (slot < 0) {
    gram_store(acc64, I, J, K, G, reinterpret_cast<float*>(&lds[0][0][0]), tid, wm, wn, lane);
    return;
  }
  // a piece: its fp64 partial tile, row-major [128][128], summed by the fix-up pass
  double* dst = partial + (int64_t)slot * kGT * kGT;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * 64 + b * 32 + (lane & 31);
        dst[row * kGT + col] = acc64[a][b][r];
      }
}

// Adds each cut tile's pieces in piece order.  Block (x + 8 l, y) takes rows
// 8 y .. 8 y + 7 of XCD x's l-th cut tile; a thread sums 4 adjacent elements
// and writes them to G, and off the diagonal to the mirrored column.
__global__ __launch_bounds__(256) void gram_fixup_kernel(const double* __restrict__ partial, int64_t K,
                                                         float* __restrict__ G, GramPlan plan) {
  const int x = (int)(blockIdx.x & 7), l = (int)(blockIdx.x >> 3);
  if (l >= plan.left[x]) return;
  int I, J;
  if (!gram_tile(x, plan.full[x] + l, (int)(K / kGT), I, J)) return;
  const int S = plan.pieces[x];
  const int row = (int)blockIdx.y * kGramStrip + (int)(threadIdx.x >> 5), col = 4 * (int)(threadIdx.x & 31);
  const double* src = partial + (int64_t)(plan.piece_base[x] + l * S) * kGT * kGT + row * kGT + col;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int p = 0; p < S; ++p) acc += *reinterpret_cast<const f64x4*>(src + (int64_t)p * kGT * kGT);
  const int64_t r0 = (int64_t)I * kGT, c0 = (int64_t)J * kGT;
  *reinterpret_cast<f32x4*>(G + (r0 + row) * K + c0 + col) = {(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
  if (I != J) {
#pragma unroll
    for (int i = 0; i < 4; ++i) G[(c0 + col + i) * K + r0 + row] = (float)acc[i];
  }
}

hipError_t launch_gram(const void* Xt, int64_t Mp, int64_t K, float* G, double* partial, hipStream_t st) {
  const GramPlan plan = gram_plan(K, Mp);
  if (plan.piece_slots > 0 && partial == nullptr) return hipErrorInvalidValue;
  gram_kernel<kGStages><<<dim3((unsigned)(8 * plan.blocks_per_xcd)), dim3(256), 0, st>>>(
      reinterpret_cast<const f16*>(Xt), Mp, K, G, partial, plan);
  if (plan.piece_slots == 0) return hipGetLastError();
  gram_fixup_kernel<<<dim3((unsigned)(8 * plan.fixup_per_xcd), kGT / kGramStrip), dim3(256), 0, st>>>(partial, K, G,
                                                                                                        plan);
  return hipGetLastError();
}

}  // namespace awq
