// W4A16 GEMM for M > 16 rows on the fp16 matrix cores.
//
// With more activation rows each weight is reused M times and the product
// turns compute-bound ("AWQ: Activation-aware Weight Quantization for On-Device
// LLM Compression and Acceleration", fdeinterviews.com/papers/awq, paragraph 9:
// under large batches serving becomes more compute-bound).  Each block stages
// one 128-channel group of its weight rows, dequantizes it once into LDS as
// fp16 w_hat = fp16((code - zero) * scale), stages the matching x tile, and
// runs v_mfma_f32_16x16x32_f16 over it with fp32 accumulation.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kBM = 64, kBN = 64;
constexpr int kLdsStride = kGroup + 8;  // halfs per LDS row (16-byte aligned, staggers banks)

// Block: 256 threads = 4 waves in 2x2; each wave a 32x32 quarter of the 64x64
// output tile as 2x2 MFMA tiles.  MFMA layouts: A lane l holds
// A[l%16][8*(l/16) .. +8] (x rows), B lane l holds B[8*(l/16) .. +8][l%16]
// (w_hat rows), D register r of lane l is D[4*(l/16)+r][l%16] = y[m][n].
__global__ __launch_bounds__(256) void gemm_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                   const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                   f16* __restrict__ y, int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) f16 As[kBM][kLdsStride];
  __shared__ __attribute__((aligned(16))) f16 Bs[kBN][kLdsStride];
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

  for (int64_t g = 0; g < G; ++g) {
    const int64_t k0 = g * kGroup;
    uint4 xv[4];
    uint4 wv = make_uint4(0u, 0u, 0u, 0u);
    f16 sc = (f16)0.0f;
    uint32_t z = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      xv[u] = xlive ? reinterpret_cast<const uint4*>(x + (m0 + lr) * K + k0 + lq * 32)[u] : make_uint4(0u, 0u, 0u, 0u);
    if (wlive) {
      wv = *reinterpret_cast<const uint4*>(packed + (n0 + lr) * K8 + g * 16 + lq * 4);
      sc = scales[(n0 + lr) * G + g];
      z = zero_of(zeros + (n0 + lr) * P, (int)g);
    }
    // dequantize 32 codes: w_hat = (code - zero) * scale, one fp16 rounding
    const f16x2 zb = zero_biased(z);
    const f16x2 sc2 = f16x2{sc, sc};
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
    uint32_t wh[16];
#pragma unroll
    for (int wi2 = 0; wi2 < 4; ++wi2)
#pragma unroll
      for (int j = 0; j < 4; ++j) wh[wi2 * 4 + j] = as_u32((pair_biased(words[wi2], j) - zb) * sc2);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      reinterpret_cast<uint4*>(&As[lr][lq * 32])[u] = xv[u];
      reinterpret_cast<uint4*>(&Bs[lr][lq * 32])[u] = make_uint4(wh[4 * u], wh[4 * u + 1], wh[4 * u + 2], wh[4 * u + 3]);
    }
    __syncthreads();
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
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
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

// Larger M: 128 x 96 block tiles (4 waves as 2 x 2, each 64 x 48 = 4 x 3 MFMA
// tiles), one 128-channel group per K step, LDS double-buffered so that one
// barrier per step separates the writes of step g+1 from the reads of step g,
// and the global loads of step g+1 are issued before the matrix-core work of
// step g.  At M = 256, N = 11008 the grid is 2 x 115 = 230 blocks, one per
// compute unit.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_big_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                       const f16* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros, f16* __restrict__ y,
                                                       int64_t M, int64_t N, int64_t K) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr int ACH = BM * 16 / 256;        // 16-byte chunks of the x tile per thread
  constexpr int BCH = BN * 4;               // 16-byte chunks of the packed tile
  constexpr int BCT = (BCH + 255) / 256;    // per thread
  __shared__ __attribute__((aligned(16))) f16 As[2][BM][kLdsStride];
  __shared__ __attribute__((aligned(16))) f16 Bs[2][BN][kLdsStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t K8 = K / 8, G = K / kGroup, P = (G + 1) / 2;

  uint4 ar[ACH];
  uint4 br[BCT];
  f16 bsc[BCT];
  uint32_t bz[BCT];

  auto load_stage = [&](int64_t g) {
    const int64_t k0 = g * kGroup;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + 256 * i, row = q >> 4, c16 = q & 15;
      const int64_t m = m0 + row;
      ar[i] = (m < M) ? *reinterpret_cast<const uint4*>(x + m * K + k0 + c16 * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < BCT; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 2, quarter = q & 3;
      const int64_t n = n0 + row;
      if (q < BCH && n < N) {
        br[i] = *reinterpret_cast<const uint4*>(packed + n * K8 + g * 16 + quarter * 4);
        bsc[i] = scales[n * G + g];
        bz[i] = zero_of(zeros + n * P, (int)g);
      } else {
        br[i] = make_uint4(0u, 0u, 0u, 0u);
        bsc[i] = (f16)0.0f;
        bz[i] = 0u;
      }
    }
  };
  auto store_stage = [&](int b) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + 256 * i, row = q >> 4, c16 = q & 15;
      *reinterpret_cast<uint4*>(&As[b][row][c16 * 8]) = ar[i];
    }
#pragma unroll
    for (int i = 0; i < BCT; ++i) {
      const int q = tid + 256 * i;
      if (q < BCH) {
        const int row = q >> 2, quarter = q & 3;
        const f16x2 zb = zero_biased(bz[i]);
        const f16x2 sc2 = f16x2{bsc[i], bsc[i]};
        const uint32_t words[4] = {br[i].x, br[i].y, br[i].z, br[i].w};
        uint32_t wh[16];
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int j = 0; j < 4; ++j) wh[w * 4 + j] = as_u32((pair_biased(words[w], j) - zb) * sc2);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          reinterpret_cast<uint4*>(&Bs[b][row][quarter * 32])[u] =
              make_uint4(wh[4 * u], wh[4 * u + 1], wh[4 * u + 2], wh[4 * u + 3]);
      }
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  lds_barrier();
  for (int64_t g = 0; g < G; ++g) {
    const int cur = (int)(g & 1);
    if (g + 1 < G) load_stage(g + 1);
#pragma unroll
    for (int kk = 0; kk < kGroup; kk += 32) {
      f16x8 av[TM], bv[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        av[a] = *reinterpret_cast<const f16x8*>(&As[cur][wm * WM + a * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bv[b] = *reinterpret_cast<const f16x8*>(&Bs[cur][wn * WN + b * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (g + 1 < G) store_stage(cur ^ 1);
    lds_barrier();
  }

#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * WM + a * 16 + 4 * (lane >> 4) + r;
        const int64_t n = n0 + wn * WN + b * 16 + (lane & 15);
        if (m < M && n < N) y[m * N + n] = (f16)acc[a][b][r];
      }
}

// Large M, main kernel: 128 x 128 block tiles, 4 waves in 2 x 2, each wave a
// 64 x 64 tile of 2 x 2 v_mfma_f32_32x32x16_f16 (the 32-wide form sustains
// about twice the throughput of the 16-wide one with one wave per SIMD).  One
// 128-channel group per K step; LDS double-buffered (one barrier per step);
// global loads run two steps ahead of the matrix cores in two register sets.
// 32x32x16 layouts: A lane l holds A[l%32][8*(l/32) .. +8], B lane l holds
// B[8*(l/32) .. +8][l%32], D register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
struct Stage {
  uint4 a[8];
  uint4 b[2];
  uint16_t sc[2];  // raw fp16 bits of the group step
  uint32_t zb[2];  // raw zeros byte (two groups' nibbles)
};

// Loads of one K step.  Every load is unconditional (rows past M or N are
// clamped to the last row and masked when stored) and nothing is computed from
// a loaded value here, so no wait on the load counter is needed until the
// stage is written to LDS one step later.
__device__ __forceinline__ void g3_load(Stage& st, const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                        const f16* __restrict__ scales, const uint8_t* __restrict__ zeros, int tid,
                                        int64_t m0, int64_t n0, int64_t M, int64_t N, int64_t K, int64_t g) {
  const int64_t K8 = K / 8, G = K / kGroup, P = (G + 1) / 2, k0 = g * kGroup;
  const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(scales);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + 256 * i, row = q >> 4, c16 = q & 15;
    const int64_t m = (m0 + row < M) ? m0 + row : M - 1;
    st.a[i] = *reinterpret_cast<const uint4*>(x + m * K + k0 + c16 * 8);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i, row = q >> 2, quarter = q & 3;
    const int64_t n = (n0 + row < N) ? n0 + row : N - 1;
    st.b[i] = *reinterpret_cast<const uint4*>(packed + n * K8 + g * 16 + quarter * 4);
    st.sc[i] = sc16[n * G + g];
    st.zb[i] = zeros[n * P + (g >> 1)];
  }
}

__device__ __forceinline__ void g3_store(const Stage& st, f16 (*As)[kLdsStride], f16 (*Bs)[kLdsStride], int tid,
                                         int64_t m0, int64_t n0, int64_t M, int64_t N, int64_t g) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + 256 * i, row = q >> 4, c16 = q & 15;
    const uint4 v = (m0 + row < M) ? st.a[i] : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&As[row][c16 * 8]) = v;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i, row = q >> 2, quarter = q & 3;
    const bool live = n0 + row < N;
    const uint32_t z = (st.zb[i] >> (4 * (g & 1))) & 0xFu;
    const f16x2 zb = zero_biased(z);
    const f16 sc = live ? __builtin_bit_cast(f16, st.sc[i]) : (f16)0.0f;
    const f16x2 sc2 = f16x2{sc, sc};
    const uint32_t words[4] = {st.b[i].x, st.b[i].y, st.b[i].z, st.b[i].w};
    uint32_t wh[16];
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) wh[w * 4 + j] = as_u32((pair_biased(words[w], j) - zb) * sc2);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      reinterpret_cast<uint4*>(&Bs[row][quarter * 32])[u] = make_uint4(wh[4 * u], wh[4 * u + 1], wh[4 * u + 2], wh[4 * u + 3]);
  }
}

__device__ __forceinline__ void g3_compute(f32x16 (&acc)[2][2], const f16 (*As)[kLdsStride], const f16 (*Bs)[kLdsStride],
                                           int lane, int wm, int wn) {
#pragma unroll
  for (int kk = 0; kk < kGroup; kk += 16) {
    f16x8 av[2], bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
      av[a] = *reinterpret_cast<const f16x8*>(&As[wm * 64 + a * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      bv[b] = *reinterpret_cast<const f16x8*>(&Bs[wn * 64 + b * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void gemm_mfma32_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                          const f16* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros, f16* __restrict__ y,
                                                          int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) f16 As[2][128][kLdsStride];
  __shared__ __attribute__((aligned(16))) f16 Bs[2][128][kLdsStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * 128, n0 = (int64_t)blockIdx.x * 128;
  const int64_t G = K / kGroup;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  Stage s0, s1;
  g3_load(s0, x, packed, scales, zeros, tid, m0, n0, M, N, K, 0);
  if (G > 1) g3_load(s1, x, packed, scales, zeros, tid, m0, n0, M, N, K, 1);
  g3_store(s0, As[0], Bs[0], tid, m0, n0, M, N, 0);
  lds_barrier();
  // invariant at the top of step g: LDS buffer g&1 holds step g; the other
  // register set holds the loads of step g+1 (in flight).
  for (int64_t g = 0; g < G; g += 2) {
    // step g (LDS 0); s1 holds g+1; s0 is free
    if (g + 2 < G) g3_load(s0, x, packed, scales, zeros, tid, m0, n0, M, N, K, g + 2);
    g3_compute(acc, As[0], Bs[0], lane, wm, wn);
    if (g + 1 < G) g3_store(s1, As[1], Bs[1], tid, m0, n0, M, N, g + 1);
    lds_barrier();
    if (g + 1 >= G) break;
    // step g+1 (LDS 1); s0 holds g+2; s1 is free
    if (g + 3 < G) g3_load(s1, x, packed, scales, zeros, tid, m0, n0, M, N, K, g + 3);
    g3_compute(acc, As[1], Bs[1], lane, wm, wn);
    if (g + 2 < G) g3_store(s0, As[0], Bs[0], tid, m0, n0, M, N, g + 2);
    lds_barrier();
  }

#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + b * 32 + (lane & 31);
        if (m < M && n < N) y[m * N + n] = (f16)acc[a][b][r];
      }
}

#ifndef AWQ_GEMM_BM
#define AWQ_GEMM_BM 128
#endif
#ifndef AWQ_GEMM_BN
#define AWQ_GEMM_BN 96
#endif

hipError_t launch_gemm(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t st) {
#ifndef AWQ_GEMM_LEGACY
  if (gemm_pipe_supported(M, K)) return launch_gemm_pipe(x, packed, scales, zeros, y, M, N, K, st);
#endif
#ifndef AWQ_GEMM_OLD_BIG
  if (M > 64) {
    dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
    gemm_mfma32_kernel<<<grid, dim3(256), 0, st>>>(
        reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed),
        reinterpret_cast<const f16*>(scales), reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), M, N,
        K);
    return hipGetLastError();
  }
#endif
  if (M > 64) {
    constexpr int BM = AWQ_GEMM_BM, BN = AWQ_GEMM_BN;
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    gemm_big_kernel<BM, BN><<<grid, dim3(256), 0, st>>>(
        reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed),
        reinterpret_cast<const f16*>(scales), reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), M, N,
        K);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  gemm_kernel<<<grid, dim3(256), 0, st>>>(reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed),
                                          reinterpret_cast<const f16*>(scales), reinterpret_cast<const uint8_t*>(zeros),
                                          reinterpret_cast<f16*>(y), M, N, K);
  return hipGetLastError();
}

}  // namespace awq
