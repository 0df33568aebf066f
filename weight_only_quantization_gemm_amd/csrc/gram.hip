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
// (global_load_lds_dwordx4), four stages deep, so three stages of loads are
// in flight while the matrix cores work on the fourth.
#include "awq_common.h"
#include "awq_internal.h"
#include "mfma_pipe.h"

namespace awq {

constexpr int kGT = 128;          // tile of G
constexpr int kGStages = 4;       // pipeline depth
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
// is D[8*(r/4) + 4*(l/32) + r%4][l%32].
__global__ __launch_bounds__(256) void gram_kernel(const f16* __restrict__ Xt, int64_t Mp, int64_t K,
                                                   float* __restrict__ G) {
  __shared__ __attribute__((aligned(16))) f16 lds[kGStages][2][kGT * 64];  // 131,072 B
  const int nb = (int)(K / kGT);
  int I, J;
  if (!gram_tile((int)(blockIdx.x & 7), (int)(blockIdx.x >> 3), nb, I, J)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)I * kGT, c0 = (int64_t)J * kGT;
  const int64_t T = Mp / 64;

  auto issue = [&](int64_t t) {
    f16* a = lds[t % kGStages][0];
    f16* b = lds[t % kGStages][1];
    dl_tile<kGT, 4>(a, Xt, Mp, r0, K, t * 64, wave, lane);
    dl_tile<kGT, 4>(b, Xt, Mp, c0, K, t * 64, wave, lane);
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

  for (int64_t t = 0; t < kGStages - 1 && t < T; ++t) issue(t);
  for (int64_t t = 0; t < T; ++t) {
    // stage t must have landed: stages t+1 .. t+kGStages-2 may still be in flight
    const int64_t ahead = (T - 1 - t) < (kGStages - 2) ? (T - 1 - t) : (kGStages - 2);
    if (ahead >= 2) wait_vmcnt<2 * kGLoadsPerWave>();
    else if (ahead == 1) wait_vmcnt<kGLoadsPerWave>();
    else wait_vmcnt<0>();
    lds_barrier();  // every wave's part of stage t is in LDS; stage t-1 is no longer read
    if (t + kGStages - 1 < T) issue(t + kGStages - 1);
    const f16* A = lds[t % kGStages][0];
    const f16* B = lds[t % kGStages][1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + (lane >> 5);
      f16x8 av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = frag(A, wm * 64 + a * 32 + (lane & 31), c);
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = frag(B, wn * 64 + b * 32 + (lane & 31), c);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
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

  // Stage the tile in LDS (fp32), then write it (and its mirror) row-coalesced.
  lds_barrier();
  float* tile = reinterpret_cast<float*>(&lds[0][0][0]);  // [128][129]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * 64 + b * 32 + (lane & 31);
        tile[row * (kGT + 1) + col] = (float)acc64[a][b][r];
      }
  __syncthreads();
  for (int i = tid; i < kGT * kGT; i += 256) {
    const int ry = i >> 7, cx = i & 127;
    G[(r0 + ry) * K + c0 + cx] = tile[ry * (kGT + 1) + cx];
    if (I != J) G[(c0 + ry) * K + r0 + cx] = tile[cx * (kGT + 1) + ry];
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
  gram_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(reinterpret_cast<const f16*>(Xt), Mp, K, G);
  return hipGetLastError();
}

}  // namespace awq
