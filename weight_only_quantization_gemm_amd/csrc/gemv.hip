// W4A16 GEMV for M <= 8 activation rows: y[m][n] = sum_k x[m][k] * w_hat[n][k].
//
// Decoding reads every weight once per token and does little arithmetic with
// it, so this kernel is bound by HBM bandwidth; 4-bit codes cut that traffic
// about 4x ("AWQ: Activation-aware Weight Quantization for On-Device LLM
// Compression and Acceleration", fdeinterviews.com/papers/awq, paragraphs 1
// and 6).  Codes are dequantized on the fly in registers (OpenAlex record of
// the GetMobile AWQ article, abstract), using the packed nibble order: one
// shift and one and-or turn a word into two fp16 values 1024 + code, one
// packed fp16 subtraction gives (code - zero) exactly, and v_dot2_f32_f16
// multiplies pairs with x into an fp32 sum.  The group scale is applied in
// fp32 once per 32 codes.
//
// Mapping: a wave owns R output rows; lane l streams the 16-byte chunks
// l, l+64, ... (32 codes each, inside one 128-channel group) of every one of
// its rows, so a wave's loads of one row are 1 KB contiguous.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

typedef __fp16 h16x2 __attribute__((ext_vector_type(2)));

__device__ inline float dot2_acc(f16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, a), __builtin_bit_cast(h16x2, b), c, false);
}

template <int MB, int R>
__global__ __launch_bounds__(256) void gemv_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                   const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                   f16* __restrict__ y, int64_t N, int64_t K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * R;
  const int64_t K8 = K / 8, G = K / kGroup, P = (G + 1) / 2;
  const int64_t nchunk = K / 32;
  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[r][m] = 0.0f;

  for (int64_t c = lane; c < nchunk; c += kWave) {
    const int64_t g = c >> 2;
    uint4 xv[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[m][u] = reinterpret_cast<const uint4*>(x + m * K + c * 32)[u];
    uint4 wv[R];
    float sc[R];
    uint32_t zr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r;
      if (row < N) {
        wv[r] = *reinterpret_cast<const uint4*>(packed + row * K8 + c * 4);
        sc[r] = (float)scales[row * G + g];
        zr[r] = zero_of(zeros + row * P, (int)g);
      } else {
        wv[r] = make_uint4(0u, 0u, 0u, 0u);
        sc[r] = 0.0f;
        zr[r] = 0u;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const f16x2 zb = zero_biased(zr[r]);
      const uint32_t words[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
      float part[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) part[m] = 0.0f;
#pragma unroll
      for (int wi = 0; wi < 4; ++wi)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x2 d = pair_biased(words[wi], j) - zb;  // (code - zero), exact
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const uint32_t xw = (j == 0) ? xv[m][wi].x : (j == 1) ? xv[m][wi].y : (j == 2) ? xv[m][wi].z : xv[m][wi].w;
            part[m] = dot2_acc(d, xw, part[m]);
          }
        }
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] += sc[r] * part[m];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == 0 && row < N) y[m * N + row] = (f16)v;
    }
  }
}

template <int MB>
static hipError_t gemv_m(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                         int64_t N, int64_t K, hipStream_t st) {
  constexpr int R = (MB <= 2) ? 4 : 2;
  const int64_t rows_per_block = 4 * R;
  dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block));
  gemv_kernel<MB, R><<<grid, dim3(256), 0, st>>>(
      reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed), reinterpret_cast<const f16*>(scales),
      reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), N, K);
  return hipGetLastError();
}

hipError_t launch_gemv(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t st) {
  switch (M) {
    case 1: return gemv_m<1>(x, packed, scales, zeros, y, N, K, st);
    case 2: return gemv_m<2>(x, packed, scales, zeros, y, N, K, st);
    case 3: return gemv_m<3>(x, packed, scales, zeros, y, N, K, st);
    case 4: return gemv_m<4>(x, packed, scales, zeros, y, N, K, st);
    case 5: return gemv_m<5>(x, packed, scales, zeros, y, N, K, st);
    case 6: return gemv_m<6>(x, packed, scales, zeros, y, N, K, st);
    case 7: return gemv_m<7>(x, packed, scales, zeros, y, N, K, st);
    case 8: return gemv_m<8>(x, packed, scales, zeros, y, N, K, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
