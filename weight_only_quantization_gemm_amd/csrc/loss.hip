// Output-MSE of one alpha: L = ||X E^T||_F^2 / (M N) = sum_n E_n G E_n^T / (M N)
// with G = X^T X, E = w_hat / s - w.  The search picks the alpha whose
// quantized layer changes the layer's output least on the calibration rows
// ("AWQ: Activation-aware Weight Quantization for On-Device LLM Compression and
// Acceleration", fdeinterviews.com/papers/awq, paragraph 3: grid search over
// alpha on a small calibration set, no backpropagation).
//
// Precision plan (exact rescaling, then a 22-bit split for the fp16 matrix
// cores).  With a power of two 2^e_k per channel (e_k ~ log2 sqrt(G_kk)),
//   G'_kj = G_kj 2^(-e_k - e_j),  E'_nk = E_nk 2^(e_k),  sum_n E'_n G' E'_n^T = sum_n E_n G E_n^T
// exactly, and |G'| <= ~2 (Cauchy-Schwarz) while E' stays well inside fp16
// range.  Each of E', G' is stored as an fp16 pair hi + lo (hi = fp16(v),
// lo = fp16(v - hi)), and T = E' G' is formed on v_mfma_f32_32x32x16_f16 as
// hi.hi + hi.lo + lo.hi with fp32 accumulation (the dropped lo.lo term is
// ~2^-22 relative).  Block partial sums go to fp64 and are reduced in a fixed
// order, so the result is deterministic; it agrees with an fp64 evaluation to
// about 1e-7 relative.
//
// This Gram form is used when M >= K; for M < K see the direct form below.
//
// G is symmetric: with channels in 128-wide blocks I, J,
//   sum_n E'_n G' E'_n^T = sum_n [ sum_J E'_nJ G'_JJ E'_nJ^T + 2 sum_{I<J} E'_nI G'_IJ E'_nJ^T ],
// so a block (rows n, column block J) contracts over channel blocks I <= J
// only and doubles (exactly) its accumulator before the diagonal block.
#include "awq_common.h"
#include "awq_internal.h"
#include "mfma_pipe.h"

namespace awq {

constexpr int kLT = 128;           // block tile: 128 rows n x 128 columns j

int64_t loss_partial_count(int64_t N, int64_t K) { return ((N + kLT - 1) / kLT) * (K / kLT); }

// e_k = floor(log2(G_kk) / 2), 0 where G_kk is 0 (a channel that is zero in every row).
__global__ void channel_exponent_kernel(const float* __restrict__ G, int64_t K, int32_t* __restrict__ e) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const float d = G[k * K + k];
  e[k] = (d > 0.0f) ? (ilogbf(d) >> 1) : 0;
}

// Ghi/Glo = split of G'_kj = G_kj 2^(-e_k - e_j); the scaling is exact in fp32.
__global__ void gram_split_kernel(const float* __restrict__ G, const int32_t* __restrict__ e, int64_t K,
                                  f16* __restrict__ Ghi, f16* __restrict__ Glo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= K * K) return;
  const int64_t k = i / K, j = i - k * K;
  const float v = ldexpf(G[i], -(e[k] + e[j]));
  const f16 hi = (f16)v;
  Ghi[i] = hi;
  Glo[i] = (f16)(v - (float)hi);
}

hipError_t launch_gram_split(const float* G, int64_t K, int32_t* e, void* Ghi, void* Glo, hipStream_t st) {
  channel_exponent_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(G, K, e);
  const int64_t n = K * K;
  gram_split_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(G, e, K, reinterpret_cast<f16*>(Ghi),
                                                                              reinterpret_cast<f16*>(Glo));
  return hipGetLastError();
}

// Block: 256 threads = 4 waves in 2 x 2, each a 64 x 64 tile of 2 x 2
// v_mfma_f32_32x32x16_f16 (D register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32]).  Channels are consumed 32 at a time; the
// four operand tiles of a stage (E' hi/lo rows n, G' hi/lo rows j, 128 x 32
// each) go straight from global memory into LDS, four stages deep.
constexpr int kLKS = 32;
constexpr int kLStages = 4;
constexpr int kLLoadsPerWave = 4 * kLT / 16 / 4;  // direct loads per wave per stage

__global__ __launch_bounds__(256) void loss_partial_kernel(const f16* __restrict__ Ehi, const f16* __restrict__ Elo,
                                                           const f16* __restrict__ Ghi, const f16* __restrict__ Glo,
                                                           int64_t N, int64_t K, double* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) f16 lds[kLStages][4][kLT * kLKS];  // 131,072 B
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.y * kLT;
  const int64_t j0 = (int64_t)blockIdx.x * kLT;
  const int64_t S = (j0 + kLT) / kLKS;  // channel blocks I <= J

  auto issue = [&](int64_t s) {
    const int64_t k0 = s * kLKS;
    dl_tile32<kLT, 4>(lds[s % kLStages][0], Ehi, K, n0, N, k0, wave, lane);
    dl_tile32<kLT, 4>(lds[s % kLStages][1], Elo, K, n0, N, k0, wave, lane);
    dl_tile32<kLT, 4>(lds[s % kLStages][2], Ghi, K, j0, K, k0, wave, lane);
    dl_tile32<kLT, 4>(lds[s % kLStages][3], Glo, K, j0, K, k0, wave, lane);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // E' rows n >= N are read from row N - 1; mask their A fragments to zero.
  bool arow_live[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) arow_live[a] = n0 + wm * 64 + a * 32 + (lane & 31) < N;

  for (int64_t s = 0; s < kLStages - 1 && s < S; ++s) issue(s);
  for (int64_t s = 0; s < S; ++s) {
    const int64_t ahead = (S - 1 - s) < (kLStages - 2) ? (S - 1 - s) : (kLStages - 2);
    if (ahead >= 2) wait_vmcnt<2 * kLLoadsPerWave>();
    else if (ahead == 1) wait_vmcnt<kLLoadsPerWave>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (s + kLStages - 1 < S) issue(s + kLStages - 1);
    if (s * kLKS == j0) {  // entering the diagonal block: off-diagonal blocks count twice
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[a][b][r] *= 2.0f;
    }
    const f16* Ah = lds[s % kLStages][0];
    const f16* Al = lds[s % kLStages][1];
    const f16* Bh = lds[s % kLStages][2];
    const f16* Bl = lds[s % kLStages][3];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * h + (lane >> 5);
      f16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int row = wm * 64 + a * 32 + (lane & 31);
        const f16x8 zero8 = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        ah[a] = arow_live[a] ? frag32(Ah, row, c) : zero8;
        al[a] = arow_live[a] ? frag32(Al, row, c) : zero8;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = wn * 64 + b * 32 + (lane & 31);
        bh[b] = frag32(Bh, row, c);
        bl[b] = frag32(Bl, row, c);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a], bh[b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a], bl[b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[a], bh[b], acc[a][b], 0, 0, 0);
        }
    }
  }

  // partial = sum over the tile of E'[n][j] * T[n][j], E' = hi + lo in fp32
  double sum = 0.0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t n = n0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = j0 + wn * 64 + b * 32 + (lane & 31);
        if (n < N) {
          const float e = (float)Ehi[n * K + j] + (float)Elo[n * K + j];
          sum += (double)e * (double)acc[a][b][r];
        }
      }
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_loss_partials(const void* Ehi, const void* Elo, const void* Ghi, const void* Glo, int64_t N,
                                int64_t K, double* partial, hipStream_t st) {
  dim3 grid((unsigned)(K / kLT), (unsigned)((N + kLT - 1) / kLT));
  loss_partial_kernel<<<grid, dim3(256), 0, st>>>(
      reinterpret_cast<const f16*>(Ehi), reinterpret_cast<const f16*>(Elo), reinterpret_cast<const f16*>(Ghi),
      reinterpret_cast<const f16*>(Glo), N, K, partial);
  return hipGetLastError();
}

// Direct form for M < K (few calibration rows, where X^T X is far from full
// rank and its split would lose accuracy): L = sum_{t,n} Y_tn^2 / (M N) with
// Y = X E^T, E in fp32 and X (fp16, exact in fp32) on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  Block: 64 rows t x 64 rows n, 4 waves in 2 x 2,
// each 32 x 32 as 2 x 2 MFMA tiles; 16x16x4 fp32 layouts: A lane l holds
// A[l%16][l/16], B lane l holds B[l/16][l%16], D register r of lane l is
// D[4*(l/16)+r][l%16].
constexpr int kDT = 64, kDKS = 16;

int64_t loss_direct_partial_count(int64_t M, int64_t N) { return ((M + kDT - 1) / kDT) * ((N + kDT - 1) / kDT); }

__global__ __launch_bounds__(256) void loss_direct_kernel(const f16* __restrict__ X, const float* __restrict__ E,
                                                          int64_t M, int64_t N, int64_t K,
                                                          double* __restrict__ partial) {
  __shared__ float As[kDT][kDKS + 1];
  __shared__ float Bs[kDT][kDKS + 1];
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * kDT, n0 = (int64_t)blockIdx.x * kDT;
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  const bool alive = t0 + lr < M, blive = n0 + lr < N;
  const f16* Ap = X + (alive ? t0 + lr : M - 1) * K + lc;
  const float* Bp = E + (blive ? n0 + lr : N - 1) * K + lc;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < K; k0 += kDKS) {
    const uint2 araw = *reinterpret_cast<const uint2*>(Ap + k0);
    const float4 bv = *reinterpret_cast<const float4*>(Bp + k0);
    const f16x2 a01 = as_f16x2(araw.x), a23 = as_f16x2(araw.y);
    __syncthreads();
    As[lr][lc + 0] = alive ? (float)a01.x : 0.f;
    As[lr][lc + 1] = alive ? (float)a01.y : 0.f;
    As[lr][lc + 2] = alive ? (float)a23.x : 0.f;
    As[lr][lc + 3] = alive ? (float)a23.y : 0.f;
    Bs[lr][lc + 0] = blive ? bv.x : 0.f;
    Bs[lr][lc + 1] = blive ? bv.y : 0.f;
    Bs[lr][lc + 2] = blive ? bv.z : 0.f;
    Bs[lr][lc + 3] = blive ? bv.w : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kDKS; kk += 4) {
      float a_[2], b_[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) a_[a] = As[wi * 32 + a * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int b = 0; b < 2; ++b) b_[b] = Bs[wj * 32 + b * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_[a], b_[b], acc[a][b], 0, 0, 0);
    }
  }
  double sum = 0.0;  // rows t >= M and n >= N hold zeros
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += (double)acc[a][b][r] * (double)acc[a][b][r];
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_loss_direct(const void* X, const float* E, int64_t M, int64_t N, int64_t K, double* partial,
                              hipStream_t st) {
  dim3 grid((unsigned)((N + kDT - 1) / kDT), (unsigned)((M + kDT - 1) / kDT));
  loss_direct_kernel<<<grid, dim3(256), 0, st>>>(reinterpret_cast<const f16*>(X), E, M, N, K, partial);
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
