// G = X^T X of the calibration rows, fp64 [K][K].  It turns the search's
// output MSE ||X E^T||^2 into sum_n E_n G E_n^T, whose cost no longer grows
// with the number of calibration rows.
//
// fp16 x fp16 products are exact in fp32; the matrix cores
// (v_mfma_f32_16x16x32_f16) accumulate 256 rows at a time in fp32 and the
// partial is then added into fp64 registers, so rounding error grows with
// 256 rows, not with M.  Only tiles on or above the diagonal are computed; an
// off-diagonal tile is written twice (as itself and transposed) through LDS.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kGramTile = 64;
constexpr int kGramFlush = 8;  // MFMA k-steps (x32 rows) per fp32 partial

// Xt: fp16 [K][Mp] (rows of X^T), Mp % 64 == 0.  Block: 4 waves in 2x2, each a
// 32x32 quarter as 2x2 MFMA tiles.  16x16x32 f16 MFMA layouts: A lane l holds
// A[l%16][8*(l/16) .. +8], B lane l holds B[8*(l/16) .. +8][l%16], D register r
// of lane l is D[4*(l/16)+r][l%16].
__global__ __launch_bounds__(256) void gram_kernel(const f16* __restrict__ Xt, int64_t Mp, int64_t K,
                                                   double* __restrict__ G) {
  __shared__ double tile[kGramTile][kGramTile + 1];
  const int nb = (int)(K / kGramTile);
  int I = 0, rem = (int)blockIdx.x;
  while (rem >= nb - I) {  // row I of the upper triangle holds nb - I tiles
    rem -= nb - I;
    ++I;
  }
  const int J = I + rem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t r0 = (int64_t)I * kGramTile + wi * 32;
  const int64_t c0 = (int64_t)J * kGramTile + wj * 32;
  const int koff = 8 * (lane >> 4);
  const f16* ap[2];
  const f16* bp[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) ap[a] = Xt + (r0 + a * 16 + (lane & 15)) * Mp + koff;
#pragma unroll
  for (int b = 0; b < 2; ++b) bp[b] = Xt + (c0 + b * 16 + (lane & 15)) * Mp + koff;

  double acc64[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[a][b][r] = 0.0;

  for (int64_t t0 = 0; t0 < Mp; t0 += 32 * kGramFlush) {
    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t t1 = (t0 + 32 * kGramFlush < Mp) ? t0 + 32 * kGramFlush : Mp;
    for (int64_t t = t0; t < t1; t += 32) {
      f16x8 av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = *reinterpret_cast<const f16x8*>(ap[a] + t);
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = *reinterpret_cast<const f16x8*>(bp[b] + t);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc64[a][b][r] += (double)acc[a][b][r];
  }

  // Stage the 64x64 tile in LDS, then write it (and its mirror) row-coalesced.
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        tile[wi * 32 + a * 16 + 4 * (lane >> 4) + r][wj * 32 + b * 16 + (lane & 15)] = acc64[a][b][r];
  __syncthreads();
  const int64_t gi = (int64_t)I * kGramTile, gj = (int64_t)J * kGramTile;
  const int cx = tid & 63;
  for (int ry = tid >> 6; ry < kGramTile; ry += 4) {
    G[(gi + ry) * K + gj + cx] = tile[ry][cx];
    if (I != J) G[(gj + ry) * K + gi + cx] = tile[cx][ry];
  }
}

hipError_t launch_gram(const void* Xt, int64_t Mp, int64_t K, double* G, hipStream_t st) {
  const int64_t nb = K / kGramTile;
  const int64_t blocks = nb * (nb + 1) / 2;
  gram_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(reinterpret_cast<const f16*>(Xt), Mp, K, G);
  return hipGetLastError();
}

}  // namespace awq
