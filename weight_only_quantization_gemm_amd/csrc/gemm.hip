// W4A16 GEMM for M > 16 rows on the fp16 matrix cores: the general-shape
// path, for the K the pipelined kernel cannot hold (its LDS keeps the block's
// scales and zeros for all of K), the dispatcher for M > 16, and the product
// of the 3-bit format for M > 2.
//
// With more activation rows each weight is reused M times and the product
// turns compute-bound ("AWQ: Activation-aware Weight Quantization for On-Device
// LLM Compression and Acceleration", fdeinterviews.com/papers/awq, paragraph 9:
// under large batches serving becomes more compute-bound).  Each block stages
// one 128-channel group of its weight rows in LDS as fp16 (code - zero), exact,
// with the group's scales, stages the matching x tile, runs
// v_mfma_f32_16x16x32_f16 over the group and adds scale * partial in fp32.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kBM = 64, kBN = 64;
constexpr int kLdsStride = kGroup + 8;  // halfs per LDS row (16-byte aligned, staggers banks)

// Block: 256 threads = 4 waves in 2x2; each wave a 32x32 quarter of the 64x64
// output tile as 2x2 MFMA tiles.  MFMA layouts: A lane l holds
// A[l%16][8*(l/16) .. +8] (x rows), B lane l holds B[8*(l/16) .. +8][l%16]
// (weight rows), D register r of lane l is D[4*(l/16)+r][l%16] = y[m][n].
template <int BITS>
__global__ __launch_bounds__(256) void gemm_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                   const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                   f16* __restrict__ y, int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) f16 As[kBM][kLdsStride];
  __shared__ __attribute__((aligned(16))) f16 Bs[kBN][kLdsStride];
  __shared__ float Ss[kBN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t K8 = K / 8, G = K / kGroup, P = (G + 1) / 2;
  const int lr = tid >> 2, lq = tid & 3;  // loader row, quarter of the 128-channel group
  const bool xlive = (m0 + lr) < M, wlive = (n0 + lr) < N;

  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t bias = bias_in_vgpr();
  for (int64_t g = 0; g < G; ++g) {
    const int64_t k0 = g * kGroup;
    uint4 xv[4];
    uint32_t words[4] = {0u, 0u, 0u, 0u};  // the thread's 32 codes: 4 words (4-bit) or 3 (3-bit)
    f16 sc = (f16)0.0f;
    uint32_t z = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      xv[u] = xlive ? reinterpret_cast<const uint4*>(x + (m0 + lr) * K + k0 + lq * 32)[u] : make_uint4(0u, 0u, 0u, 0u);
    if (wlive) {
      if constexpr (BITS == 4) {
        const uint4 wv = *reinterpret_cast<const uint4*>(packed + (n0 + lr) * K8 + g * 16 + lq * 4);
        words[0] = wv.x, words[1] = wv.y, words[2] = wv.z, words[3] = wv.w;
      } else {
        const uint32_t* src = packed + ((n0 + lr) * (K / 32) + g * 4 + lq) * 3;
        words[0] = src[0], words[1] = src[1], words[2] = src[2];
      }
      sc = scales[(n0 + lr) * G + g];
      z = zero_of(zeros + (n0 + lr) * P, (int)g);
    }
    // 32 codes as fp16 (code - zero), exact: channel pair p of the chunk in wh[p]
    const f16x2 zb = zero_biased(z);
    uint32_t wh[16];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int wi2 = 0; wi2 < 4; ++wi2)
#pragma unroll
        for (int j = 0; j < 4; ++j) wh[wi2 * 4 + j] = as_u32(pair_biased(words[wi2], j, bias) - zb);
    } else {
#pragma unroll
      for (int p = 0; p < 15; ++p)
        wh[p] = as_u32(as_f16x2(((words[p / 5] >> (3 * (p % 5))) & 0x00070007u) | bias) - zb);
      const uint32_t p15 = ((words[0] >> 15) & 0x00010001u) | ((words[1] >> 14) & 0x00020002u) |
                           ((words[2] >> 13) & 0x00040004u);
      wh[15] = as_u32(as_f16x2(p15 | bias) - zb);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      reinterpret_cast<uint4*>(&As[lr][lq * 32])[u] = xv[u];
      reinterpret_cast<uint4*>(&Bs[lr][lq * 32])[u] = make_uint4(wh[4 * u], wh[4 * u + 1], wh[4 * u + 2], wh[4 * u + 3]);
    }
    if (lq == 0) Ss[lr] = (float)sc;
    __syncthreads();
    f32x4 d[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) d[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kGroup; kk += 32) {
      f16x8 av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        av[a] = *reinterpret_cast<const f16x8*>(&As[wi * 32 + a * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[b] = *reinterpret_cast<const f16x8*>(&Bs[wj * 32 + b * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) d[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bv[b], d[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float scf = Ss[wj * 32 + b * 16 + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][b][r] = fmaf(scf, d[a][b][r], acc[a][b][r]);
    }
  }

#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wi * 32 + a * 16 + 4 * (lane >> 4) + r;
        const int64_t n = n0 + wj * 32 + b * 16 + (lane & 15);
        if (m < M && n < N) y[m * N + n] = (f16)acc[a][b][r];
      }
}

hipError_t launch_gemm(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                       int64_t N, int64_t K, void* ws, hipStream_t st) {
  if (ws != nullptr && gemm_pipe_streamk(M, N, K, 4)) return launch_gemm_pipe(x, packed, scales, zeros, y, M, N, K, ws, st);
  if (ring_mid_supported(M, N, K, 4)) return launch_ring_mid(x, packed, scales, zeros, y, M, N, K, 4, st);
  if (gemv_wide_preferred(M, N, K)) return launch_gemv_wide(x, packed, scales, zeros, y, M, N, K, st);
  if (gemm_pipe_supported(M, N, K)) return launch_gemm_pipe(x, packed, scales, zeros, y, M, N, K, ws, st);
  if ((M + kBM - 1) / kBM > 65535) return hipErrorInvalidValue;  // grid.y limit
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (KernelPlan* p = active_plan()) return plan_record(p, "gemm_kernel<4> block=256 grid=%ux%u", grid.x, grid.y);
  gemm_kernel<4><<<grid, dim3(256), 0, st>>>(reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed),
                                             reinterpret_cast<const f16*>(scales),
                                             reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), M, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm3(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                        int64_t N, int64_t K, void* ws, hipStream_t st) {
  if (gemv3_supported(M, K)) return launch_gemv3(x, packed, scales, zeros, y, M, N, K, st);
  if (ring3_supported(M, N, K)) return launch_ring3(x, packed, scales, zeros, y, M, N, K, st);
  if (ws != nullptr && gemm_pipe_streamk(M, N, K, 3)) return launch_gemm_pipe3(x, packed, scales, zeros, y, M, N, K, ws, st);
  if (ring_mid_pipe_preferred(M, N, K) && gemm_pipe3_supported(M, N, K))
    return launch_gemm_pipe3(x, packed, scales, zeros, y, M, N, K, ws, st);
  if (ring_mid_supported(M, N, K, 3)) return launch_ring_mid(x, packed, scales, zeros, y, M, N, K, 3, st);
  if (gemm_pipe3_supported(M, N, K)) return launch_gemm_pipe3(x, packed, scales, zeros, y, M, N, K, ws, st);
  if ((M + kBM - 1) / kBM > 65535) return hipErrorInvalidValue;  // grid.y limit
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (KernelPlan* p = active_plan()) return plan_record(p, "gemm_kernel<3> block=256 grid=%ux%u", grid.x, grid.y);
  gemm_kernel<3><<<grid, dim3(256), 0, st>>>(reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed),
                                             reinterpret_cast<const f16*>(scales),
                                             reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), M, N, K);
  return hipGetLastError();
}

}  // namespace awq
