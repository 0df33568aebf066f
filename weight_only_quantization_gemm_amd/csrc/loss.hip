// Output-MSE of one alpha: L = ||X E^T||_F^2 / (M N) = sum_n E_n G E_n^T / (M N)
// with G = X^T X, E = w_hat / s - w (fp64).  The search picks the alpha whose
// quantized layer changes the layer's output least on the calibration rows
// ("AWQ: Activation-aware Weight Quantization for On-Device LLM Compression and
// Acceleration", fdeinterviews.com/papers/awq, paragraph 3: grid search over
// alpha on a small calibration set, no backpropagation).
//
// The contraction T = E G runs on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64); each block then forms sum(E .* T) over its tile.
// Partials are written per block and summed in a fixed order, so the result
// is deterministic.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kLossTile = 64;   // 64 (rows n) x 64 (columns j) per block
constexpr int kLossKStep = 16;  // k per LDS stage
constexpr int kLossPad = 2;     // LDS row padding (doubles)

int64_t loss_partial_count(int64_t N, int64_t K) {
  return ((N + kLossTile - 1) / kLossTile) * (K / kLossTile);
}

// Block (256 threads, 4 waves in 2x2) owns T[n0:n0+64][j0:j0+64]; each wave a
// 32x32 quarter as 2x2 MFMA tiles of 16x16.  Operand layouts of the 16x16x4
// fp64 MFMA: A lane l holds A[l%16][l/16], B lane l holds B[l/16][l%16], and
// D register r of lane l is D[l/16 + 4*r][l%16] (rows interleave across the
// four registers, unlike the fp32-output MFMAs).
__global__ __launch_bounds__(256) void loss_partial_kernel(const double* __restrict__ E, const double* __restrict__ G,
                                                           int64_t N, int64_t K, double* __restrict__ partial) {
  __shared__ double As[kLossTile][kLossKStep + kLossPad];
  __shared__ double Bs[kLossTile][kLossKStep + kLossPad];
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.y * kLossTile;
  const int64_t j0 = (int64_t)blockIdx.x * kLossTile;
  const int lr = tid >> 2, lc = (tid & 3) * 4;  // loader: row, first of 4 columns
  const bool arow_live = (n0 + lr) < N;
  const double* Ap = E + (n0 + lr) * K + lc;
  const double* Bp = G + (j0 + lr) * K + lc;  // G symmetric: B[k][j] = G[j][k]

  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

  for (int64_t k0 = 0; k0 < K; k0 += kLossKStep) {
    double2 a01 = make_double2(0.0, 0.0), a23 = make_double2(0.0, 0.0);
    if (arow_live) {
      a01 = *reinterpret_cast<const double2*>(Ap + k0);
      a23 = *reinterpret_cast<const double2*>(Ap + k0 + 2);
    }
    double2 b01 = *reinterpret_cast<const double2*>(Bp + k0);
    double2 b23 = *reinterpret_cast<const double2*>(Bp + k0 + 2);
    __syncthreads();
    As[lr][lc + 0] = a01.x; As[lr][lc + 1] = a01.y; As[lr][lc + 2] = a23.x; As[lr][lc + 3] = a23.y;
    Bs[lr][lc + 0] = b01.x; Bs[lr][lc + 1] = b01.y; Bs[lr][lc + 2] = b23.x; Bs[lr][lc + 3] = b23.y;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kLossKStep; kk += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = As[wi * 32 + a * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = Bs[wj * 32 + b * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }

  double sum = 0.0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + wi * 32 + a * 16 + (lane >> 4) + 4 * r;
        const int64_t j = j0 + wj * 32 + b * 16 + (lane & 15);
        if (n < N) sum += E[n * K + j] * acc[a][b][r];
      }
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_loss_partials(const double* E, const double* G, int64_t N, int64_t K, double* partial,
                                hipStream_t st) {
  dim3 grid((unsigned)(K / kLossTile), (unsigned)((N + kLossTile - 1) / kLossTile));
  loss_partial_kernel<<<grid, dim3(256), 0, st>>>(E, G, N, K, partial);
  return hipGetLastError();
}

// loss[0] = (sum of partial[0..count)) / mn, summed in a fixed order.
__global__ __launch_bounds__(256) void loss_reduce_kernel(const double* __restrict__ partial, int64_t count,
                                                          double mn, double* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += 256) s += partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = red[0] / mn;
}

hipError_t launch_loss_reduce(const double* partial, int64_t count, double mn, double* loss, hipStream_t st) {
  loss_reduce_kernel<<<dim3(1), dim3(256), 0, st>>>(partial, count, mn, loss);
  return hipGetLastError();
}

// First index of the smallest loss.
__global__ void argmin_kernel(const double* __restrict__ loss, int n, int32_t* __restrict__ best) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int b = 0;
  for (int i = 1; i < n; ++i)
    if (loss[i] < loss[b]) b = i;
  best[0] = b;
}

hipError_t launch_argmin(const double* loss, int n, int32_t* best, hipStream_t st) {
  argmin_kernel<<<dim3(1), dim3(64), 0, st>>>(loss, n, best);
  return hipGetLastError();
}

}  // namespace awq
