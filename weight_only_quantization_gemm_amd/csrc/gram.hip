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
void gram_kernel(const f16* __restrict__ Xt, int64_t Mp, int64_t K, float* __restrict__ G) {
  constexpr int D = STAGES - 1;  // stages in flight ahead of the one computed
  __shared__ __attribute__((aligned(16))) f16 lds[STAGES][2][kGT * 64];
  const int nb = (int)(K / kGT);
  int I, J;
  if (!gram_tile((int)(blockIdx.x & 7), (int)(blockIdx.x >> 3), nb, I, J)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)I * kGT, c0 = (int64_t)J * kGT;
  const int T = (int)(Mp / 64);

  TilePlan<kGT, 4, 64> pa, pb;
  pa.init(Xt, Mp, r0, K, wave, lane);
  pb.init(Xt, Mp, c0, K, wave, lane);
  auto issue = [&](int t, int slot) {
    const int64_t k0 = (int64_t)(t < T ? t : T - 1) * 64;
    pa.issue(lds[slot][0], k0);
    pb.issue(lds[slot][1], k0);
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

  for (int t = 0; t < D; ++t) issue(t, t);
  int cur = 0, nxt = D;  // ring slots of stage t and of stage t + D
  for (int t = 0; t < T; ++t) {
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

  // Stage the tile in LDS (fp32) 64 rows at a time, then write those rows (and,
  // off the diagonal, the mirrored columns) row-coalesced.
  float* tile = reinterpret_cast<float*>(&lds[0][0][0]);  // [64][129]
  static_assert(STAGES * 2 * kGT * 64 * 2 >= 64 * (kGT + 1) * 4, "the fp32 half tile must fit the stage buffers");
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lds_barrier();  // the stage buffers (or the previous half) are no longer read
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

hipError_t launch_gram(const void* Xt, int64_t Mp, int64_t K, float* G, hipStream_t st) {
  const int nb = (int)(K / kGT), ns = gram_super_tiles(nb);
  int per[8] = {0, 0, 0, 0, 0, 0, 0, 0}, s = 0;
  for (int si = 0; si < ns; ++si)
    for (int sj = si; sj < ns; ++sj, ++s) per[s % 8] += gram_super_count(si, sj, nb);
  int most = 0;
  for (int x = 0; x < 8; ++x) most = per[x] > most ? per[x] : most;
  const int64_t blocks = 8 * (int64_t)most;
  gram_kernel<kGStages><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(reinterpret_cast<const f16*>(Xt), Mp, K, G);
  return hipGetLastError();
}

}  // namespace awq
