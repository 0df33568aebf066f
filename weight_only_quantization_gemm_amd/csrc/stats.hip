// Calibration statistics: per-channel mean |x| (exact), and the transposed
// copy of the calibration rows that the Gram kernel reads.
//
// AWQ derives each channel's scale from the channel's average activation
// magnitude and collects nothing but such statistics from the calibration set
// ("AWQ: Activation-aware Weight Quantization for On-Device LLM Compression and
// Acceleration", fdeinterviews.com/papers/awq, paragraphs 3 and 7).
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

// Rows summed per thread before the partial goes to the 64-bit integer total.
// Each fp16 |x| is below 2^16 and a multiple of 2^-24; a sum of at most 2^13 of
// them is a multiple of 2^-24 below 2^29, which fp64 (53-bit significand)
// represents exactly, so the fp64 partial is exact in any order.
constexpr int kStatsRows = 256;
constexpr int kStatsThreads = 256;

__global__ void fill_u64_kernel(unsigned long long* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__global__ __launch_bounds__(kStatsThreads) void stats_accumulate_kernel(
    const uint4* __restrict__ X, int64_t M, int64_t K8, unsigned long long* __restrict__ S) {
  const int64_t c = (int64_t)blockIdx.x * kStatsThreads + threadIdx.x;  // 8-channel chunk
  if (c >= K8) return;
  const int64_t t0 = (int64_t)blockIdx.y * kStatsRows;
  const int64_t t1 = (t0 + kStatsRows < M) ? t0 + kStatsRows : M;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  const uint4* p = X + t0 * K8 + c;
  int64_t t = t0;
  for (; t + 4 <= t1; t += 4) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[u * K8];
    p += 4 * K8;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x2 h = as_f16x2(w[i] & 0x7FFF7FFFu);  // |x| by clearing the sign bits
        acc[2 * i] += (double)(float)h.x;
        acc[2 * i + 1] += (double)(float)h.y;
      }
    }
  }
  for (; t < t1; ++t) {
    uint4 v = *p;
    p += K8;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x2 h = as_f16x2(w[i] & 0x7FFF7FFFu);
      acc[2 * i] += (double)(float)h.x;
      acc[2 * i + 1] += (double)(float)h.y;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // exact: acc is an integer multiple of 2^-24 below 2^29
    unsigned long long units = (unsigned long long)(acc[i] * 16777216.0);
    if (units) atomicAdd(S + c * 8 + i, units);
  }
}

// a[k] = S[k] * 2^-24 / M, in place (S and a share storage).
__global__ void stats_finalize_kernel(double* a, int64_t K, int64_t M) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  unsigned long long s = reinterpret_cast<unsigned long long*>(a)[k];
  a[k] = (double)s * 0x1p-24 / (double)M;
}

hipError_t launch_channel_mean_abs(const void* X, int64_t M, int64_t K, double* a, hipStream_t st) {
  const int64_t K8 = K / 8;
  unsigned long long* S = reinterpret_cast<unsigned long long*>(a);
  fill_u64_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(S, K);
  dim3 grid((unsigned)((K8 + kStatsThreads - 1) / kStatsThreads), (unsigned)((M + kStatsRows - 1) / kStatsRows));
  stats_accumulate_kernel<<<grid, dim3(kStatsThreads), 0, st>>>(reinterpret_cast<const uint4*>(X), M, K8, S);
  stats_finalize_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(a, K, M);
  return hipGetLastError();
}

// Xt[k][t] = X[t][k] for t < M, 0 for M <= t < Mp (Mp a multiple of 64).
// 64 x 64 tiles through LDS, 16 bytes per global access: a thread reads 8
// channels of one row t (eight threads cover a row's 128 bytes) and writes 8
// rows t of one channel k.  The LDS row pitch of 66 halfs puts the eight rows a
// write gathers from (t = 8c .. 8c + 7 for the eight c of a wave) on distinct
// banks; the row is stored as four 4-byte words (its 132-byte pitch is not
// 16-byte aligned).  A row chunk past K (K % 8 == 0) or past M reads zeros.
constexpr int kTP = 66;  // LDS pitch of the transpose tile, in halfs

__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t Mp, uint16_t* __restrict__ Xt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kTP];
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int64_t k0 = (int64_t)blockIdx.y * 64;
  const int c = threadIdx.x & 7, r = threadIdx.x >> 3;  // 8 chunks x 32 rows
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = r + 32 * h;
    const int64_t t = t0 + rr, k = k0 + 8 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t < M && k < K) v = *reinterpret_cast<const uint4*>(X + t * K + k);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + rr * kTP + 8 * c);
    dst[0] = v.x;
    dst[1] = v.y;
    dst[2] = v.z;
    dst[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = r + 32 * h;  // channel within the tile; this thread writes rows 8c .. 8c + 7
    const int64_t k = k0 + kk;
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = (uint32_t)tile[(8 * c + 2 * u) * kTP + kk] | ((uint32_t)tile[(8 * c + 2 * u + 1) * kTP + kk] << 16);
    if (k < K) *reinterpret_cast<uint4*>(Xt + k * Mp + t0 + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose(const void* X, int64_t M, int64_t K, int64_t Mp, void* Xt, hipStream_t st) {
  dim3 grid((unsigned)(Mp / 64), (unsigned)((K + 63) / 64));
  transpose_kernel<<<grid, dim3(256), 0, st>>>(reinterpret_cast<const uint16_t*>(X), M, K, Mp,
                                               reinterpret_cast<uint16_t*>(Xt));
  return hipGetLastError();
}

}  // namespace awq
