// W4A16 GEMV on the vector ALUs for M <= 2 activation rows (decode):
// y[m][n] = sum_k x[m][k] * w_hat[n][k].
//
// Decoding reads every weight once per token and does little arithmetic with
// it, so this kernel is bound by HBM bandwidth; 4-bit codes cut that traffic
// about 4x ("AWQ: Activation-aware Weight Quantization for On-Device LLM
// Compression and Acceleration", fdeinterviews.com/papers/awq, paragraphs 1
// and 6).  Codes are dequantized on the fly in registers (OpenAlex record of
// the GetMobile AWQ article, abstract).
//
// Arithmetic: every product is exact and the zero point is subtracted per
// code.  OR-ing a 4-bit field into the mantissa of fp16 1024.0 (0x6400) gives
// 1024 + code; a field that sits 4 bits higher gives 1024 + 16 code (still
// below 2048, where the fp16 spacing is 1).  The packed nibble order puts
// channels 2j and 2j + 1 of a word in bits 4j and 16 + 4j, so with one shift
// (w8 = w >> 8) the four channel pairs of a word are w & 0x000F000F (code
// units), w & 0x00F000F0 (16 code units) and the same two masks of w8, each
// OR-ed with the bias in one and-or.  One packed fp16 subtraction of
// (1024 + zero) or (1024 + 16 zero) leaves (code - zero) or 16 (code - zero),
// exact, and v_dot2_f32_f16 multiplies each pair with x exactly in fp32 (an
// fp16 times an integer below 2^8).  Two fp32 sums (code and 16 code units)
// are combined with the exact factor 1/16, and the group scale multiplies the
// 32-code partial sum in fp32.  A row whose codes all equal their zero points
// therefore gives exactly 0.
//
// Mapping: a block owns R output rows and spans all of K; lane l of wave w
// owns the 16-byte chunk c = 64 w + l (32 codes) of each of the R rows, so
// every wave-wide load is 1 KB of one row, contiguous.  The rows' base
// addresses are wave-uniform and each lane adds a 32-bit offset.  Each lane
// issues all of its loads (R weight chunks, their scales and zero points, and
// its 64 B of x per activation row) before the first use, so a block makes a
// single round trip to memory.  A lane's x chunk serves its R rows: the x
// bytes a block moves from L2 are 4 / R times its weight bytes.  Partial sums
// are reduced across the wave with DPP and across the block's waves through
// LDS in a fixed order.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

typedef __fp16 h16x2 __attribute__((ext_vector_type(2)));

__device__ inline float dot2_acc(f16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, a), __builtin_bit_cast(h16x2, b), c, false);
}

// DPP add: v + v[permuted lane]; lanes whose source row is masked off add 0.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float v) {
  const int src = __builtin_bit_cast(int, v);
  const int moved = __builtin_amdgcn_update_dpp(0, src, CTRL, ROW_MASK, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over the 64 lanes; the total lands in lane 63.
__device__ inline float wave_sum_to_lane63(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror: 8-lane sums
  v = dpp_add<0x140, 0xF>(v);  // row_mirror: 16-lane row sums
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

constexpr int kMaxWaves = 16;

// Waves per block: one 64-lane wave per 2048 channels (a lane takes 32).
__host__ __device__ inline int gemv_waves(int64_t K) {
  const int64_t w = (K / 32 + kWave - 1) / kWave;
  return w < 1 ? 1 : (int)w;
}

// K <= 32768 (at most 1024 chunks) keeps a block within 16 waves.
template <int MB, int R>
__global__ __launch_bounds__(1024) void gemv_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                    const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                    f16* __restrict__ y, int N, int K) {
  __shared__ float red[kMaxWaves][R * MB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = gemv_waves(K);  // == blockDim.x / 64, from the arguments (all preloaded)
  const uint32_t nchunk = (uint32_t)K / 32, G = (uint32_t)K / kGroup, P = (G + 1) / 2;
  const int row0 = blockIdx.x * R;

  // A chunk past the end of the row (last wave) reloads the row's last chunk
  // and is dropped from the sum; rows past N reload row N - 1 and are never
  // stored.
  const uint32_t c0 = (uint32_t)(wave * kWave + lane);
  const bool live = c0 < nchunk;
  const uint32_t c = live ? c0 : nchunk - 1, g = c >> 2;
  const u32x4* wrow[R];
  const uint16_t* srow[R];
  const uint8_t* zrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < N ? row0 + r : N - 1;
    wrow[r] = reinterpret_cast<const u32x4*>(packed + row * (K / 8));
    srow[r] = reinterpret_cast<const uint16_t*>(scales) + row * G;
    zrow[r] = zeros + row * P;
  }

  // All loads are issued before the first wait: the rows' scales and zero
  // points, x, then the weight chunks.  The scheduling barrier stops the
  // compiler from sinking any of them below a wait, which would add a second
  // round trip to memory (measured: up to 18% faster at M = 2 on the 7B/70B
  // shapes than the order the compiler picked by itself).
  uint32_t sr[R], zr[R];
  uint4 xv[MB][4];
  u32x4 wv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    sr[r] = srow[r][g];
    zr[r] = zrow[r][g >> 1];
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int u = 0; u < 4; ++u) xv[m][u] = reinterpret_cast<const uint4*>(x + (int64_t)m * K)[c * 4 + u];
#pragma unroll
  for (int r = 0; r < R; ++r) wv[r] = __builtin_nontemporal_load(wrow[r] + c);
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t bias = bias_in_vgpr();
  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t z = (zr[r] >> (4 * (g & 1))) & 0xFu;
    const f16x2 zb1 = as_f16x2(0x64006400u | z | (z << 16));           // (1024 + z) pair
    const f16x2 zb16 = as_f16x2(0x64006400u | (z << 4) | (z << 20));  // (1024 + 16 z) pair
    const uint32_t words[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
    float lo[MB], hi[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) lo[m] = hi[m] = 0.0f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      const uint32_t w = words[wi], w8 = w >> 8;
      const f16x2 p0 = as_f16x2((w & 0x000F000Fu) | bias) - zb1;    // channels 0, 1: code - zero
      const f16x2 p1 = as_f16x2((w & 0x00F000F0u) | bias) - zb16;   // channels 2, 3: 16 (code - zero)
      const f16x2 p2 = as_f16x2((w8 & 0x000F000Fu) | bias) - zb1;   // channels 4, 5
      const f16x2 p3 = as_f16x2((w8 & 0x00F000F0u) | bias) - zb16;  // channels 6, 7
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        lo[m] = dot2_acc(p0, xv[m][wi].x, lo[m]);
        hi[m] = dot2_acc(p1, xv[m][wi].y, hi[m]);
        lo[m] = dot2_acc(p2, xv[m][wi].z, lo[m]);
        hi[m] = dot2_acc(p3, xv[m][wi].w, hi[m]);
      }
    }
    const float sc = (float)as_f16x2(sr[r]).x;
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[r][m] = live ? sc * fmaf(hi[m], 0.0625f, lo[m]) : 0.0f;
  }

  if (nwaves == 1) {  // the whole row is in this wave: no cross-wave step
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float v = wave_sum_to_lane63(acc[r][m]);
        if (lane == 63 && row0 + r < N) y[(int64_t)m * N + row0 + r] = (f16)v;
      }
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float v = wave_sum_to_lane63(acc[r][m]);
      if (lane == 63) red[wave][r * MB + m] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < R * MB) {
    const int r = threadIdx.x / MB, m = threadIdx.x % MB;
    float v = 0.0f;
    for (int w = 0; w < nwaves; ++w) v += red[w][threadIdx.x];
    if (row0 + r < N) y[(int64_t)m * N + row0 + r] = (f16)v;
  }
}

template <int MB, int R>
static hipError_t gemv_launch(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                              int64_t N, int64_t K, hipStream_t st) {
  const int waves = gemv_waves(K);
  if (waves > kMaxWaves) return hipErrorInvalidValue;
  dim3 grid((unsigned)((N + R - 1) / R));
  if (KernelPlan* p = active_plan())
    return plan_record(p, "gemv_kernel<%d,%d> block=%d grid=%u", MB, R, waves * kWave, grid.x);
  gemv_kernel<MB, R><<<grid, dim3(waves * kWave), 0, st>>>(
      reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed), reinterpret_cast<const f16*>(scales),
      reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), (int)N, (int)K);
  return hipGetLastError();
}

// M = 1, and M = 2 on rows shorter than 16384 channels: every further
// activation row costs 4 more dot2 per packed word and the kernel turns
// VALU-bound (measured at M = 3..8 on the 7B/70B shapes: 1.1-2.4x slower than
// the matrix-core kernel; at M = 2 the matrix-core ring kernel is faster on
// long rows, 28672 x 8192 at 29 us against 36, and slower on the others, 8192
// x 28672 at 31 us against 27).
bool gemv_dot2_supported(int64_t M, int64_t K) {
  return (M == 1 || (M == 2 && K < 16384)) && K / 32 <= (int64_t)kMaxWaves * kWave;
}

// Rows per block, measured on the Llama-2 7B/70B decode shapes: 8 when both K
// and N are >= 8192 (x, reloaded per block, then costs half as much L2
// traffic; 8192 x 8192 at 8.3 us against 8.6 us with 4, 28672 x 8192 at
// 26.4 us against 27.4 us), and for two activation rows on the widest K = 4096
// layer; 4 elsewhere, which keeps more blocks in flight (4096 x 11008 at
// 6.1 us and 11008 x 4096 at 6.8 us, against 6.8 and 7.2 us with 8).  More
// chunks per lane (fewer waves) measured slower on every shape.
template <int MB>
static hipError_t gemv_rows_launch(const void* x, const void* packed, const void* scales, const void* zeros,
                                   void* y, int64_t N, int64_t K, hipStream_t st) {
  if ((K >= 8192 && N >= 8192) || (MB == 2 && N >= 16384))
    return gemv_launch<MB, 8>(x, packed, scales, zeros, y, N, K, st);
  return gemv_launch<MB, 4>(x, packed, scales, zeros, y, N, K, st);
}

// 3-bit format (three words per 32 channels of a row; see the packer).  The
// same mapping as above: lane l of wave w owns the chunk c = 64 w + l of each
// of R rows, now 12 bytes.  In a 16-bit half, fields 0, 1, 2 (bits 0-2, 3-5,
// 6-8) OR-ed into fp16 1024.0 give 1024 + q, 1024 + 8 q and 1024 + 64 q (all
// below 2048, so exact), and fields 3, 4 the same way after one shift by 9;
// the pair in the spare bits takes three shifts and ANDs.  Subtracting
// (1024 + z), (1024 + 8 z) or (1024 + 64 z) leaves the exact (q - z) times 1,
// 8 or 64, and three fp32 sums are combined with exact power-of-two factors,
// as in the 4-bit kernel.  Pair p of the chunk multiplies x word p.
template <int MB, int R>
__global__ __launch_bounds__(1024) void gemv3_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                     const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                     f16* __restrict__ y, int N, int K) {
  __shared__ float red[kMaxWaves][R * MB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = gemv_waves(K);  // == blockDim.x / 64
  const uint32_t nchunk = (uint32_t)K / 32, G = (uint32_t)K / kGroup, P = (G + 1) / 2;
  const int row0 = blockIdx.x * R;

  const uint32_t c0 = (uint32_t)(wave * kWave + lane);
  const bool live = c0 < nchunk;
  const uint32_t c = live ? c0 : nchunk - 1, g = c >> 2;
  const uint32_t* wrow[R];
  const uint16_t* srow[R];
  const uint8_t* zrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < N ? row0 + r : N - 1;
    wrow[r] = packed + row * (int64_t)(nchunk * 3);
    srow[r] = reinterpret_cast<const uint16_t*>(scales) + row * G;
    zrow[r] = zeros + row * P;
  }
  uint32_t sr[R], zr[R], wv[R][3];
  uint4 xv[MB][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    sr[r] = srow[r][g];
    zr[r] = zrow[r][g >> 1];
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int u = 0; u < 4; ++u) xv[m][u] = reinterpret_cast<const uint4*>(x + (int64_t)m * K)[c * 4 + u];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < 3; ++t) wv[r][t] = __builtin_nontemporal_load(wrow[r] + 3 * c + t);
  __builtin_amdgcn_sched_barrier(0);  // every load before the first wait, as in the 4-bit kernel

  const uint32_t bias = bias_in_vgpr();
  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t z = (zr[r] >> (4 * (g & 1))) & 0xFu;
    const f16x2 zb1 = as_f16x2(0x64006400u | z | (z << 16));           // (1024 + z) pair
    const f16x2 zb8 = as_f16x2(0x64006400u | (z << 3) | (z << 19));    // (1024 + 8 z) pair
    const f16x2 zb64 = as_f16x2(0x64006400u | (z << 6) | (z << 22));  // (1024 + 64 z) pair
    float a1[MB], a8[MB], a64[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) a1[m] = a8[m] = a64[m] = 0.0f;
    auto xword = [&](int m, int p) -> uint32_t {
      const uint4 v = xv[m][p >> 2];
      return (p & 3) == 0 ? v.x : (p & 3) == 1 ? v.y : (p & 3) == 2 ? v.z : v.w;
    };
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const uint32_t w = wv[r][t], w9 = w >> 9;
      const f16x2 p0 = as_f16x2((w & 0x00070007u) | bias) - zb1, p1 = as_f16x2((w & 0x00380038u) | bias) - zb8;
      const f16x2 p2 = as_f16x2((w & 0x01C001C0u) | bias) - zb64, p3 = as_f16x2((w9 & 0x00070007u) | bias) - zb1;
      const f16x2 p4 = as_f16x2((w9 & 0x00380038u) | bias) - zb8;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        a1[m] = dot2_acc(p0, xword(m, 5 * t), a1[m]);
        a8[m] = dot2_acc(p1, xword(m, 5 * t + 1), a8[m]);
        a64[m] = dot2_acc(p2, xword(m, 5 * t + 2), a64[m]);
        a1[m] = dot2_acc(p3, xword(m, 5 * t + 3), a1[m]);
        a8[m] = dot2_acc(p4, xword(m, 5 * t + 4), a8[m]);
      }
    }
    const f16x2 p15 = as_f16x2(((wv[r][0] >> 15) & 0x00010001u) | ((wv[r][1] >> 14) & 0x00020002u) |
                               ((wv[r][2] >> 13) & 0x00040004u) | bias) - zb1;
    const float sc = (float)as_f16x2(sr[r]).x;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      a1[m] = dot2_acc(p15, xword(m, 15), a1[m]);
      const float t = fmaf(a64[m], 0.015625f, fmaf(a8[m], 0.125f, a1[m]));  // sum x (q - z)
      acc[r][m] = live ? sc * t : 0.0f;
    }
  }

  if (nwaves == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float v = wave_sum_to_lane63(acc[r][m]);
        if (lane == 63 && row0 + r < N) y[(int64_t)m * N + row0 + r] = (f16)v;
      }
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float v = wave_sum_to_lane63(acc[r][m]);
      if (lane == 63) red[wave][r * MB + m] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < R * MB) {
    const int r = threadIdx.x / MB, m = threadIdx.x % MB;
    float v = 0.0f;
    for (int w = 0; w < nwaves; ++w) v += red[w][threadIdx.x];
    if (row0 + r < N) y[(int64_t)m * N + row0 + r] = (f16)v;
  }
}

template <int MB, int R>
static hipError_t gemv3_launch(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                               int64_t N, int64_t K, hipStream_t st) {
  const int waves = gemv_waves(K);
  if (waves > kMaxWaves) return hipErrorInvalidValue;
  if (KernelPlan* p = active_plan())
    return plan_record(p, "gemv3_kernel<%d,%d> block=%d grid=%u", MB, R, waves * kWave, (unsigned)((N + R - 1) / R));
  gemv3_kernel<MB, R><<<dim3((unsigned)((N + R - 1) / R)), dim3(waves * kWave), 0, st>>>(
      reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed), reinterpret_cast<const f16*>(scales),
      reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), (int)N, (int)K);
  return hipGetLastError();
}

bool gemv3_supported(int64_t M, int64_t K) { return gemv_dot2_supported(M, K); }

// Rows per block as for the 4-bit kernel (measured the same way: 8 rows win on
// 8192 x 8192 and wider, 7.4 us against 7.7 us, 4 rows below, 3.8 us against
// 4.5 us at 4096 x 4096).
hipError_t launch_gemv3(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                        int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const bool wide = (K >= 8192 && N >= 8192) || (M == 2 && N >= 16384);
  if (M == 1)
    return wide ? gemv3_launch<1, 8>(x, packed, scales, zeros, y, N, K, st)
                : gemv3_launch<1, 4>(x, packed, scales, zeros, y, N, K, st);
  if (M == 2)
    return wide ? gemv3_launch<2, 8>(x, packed, scales, zeros, y, N, K, st)
                : gemv3_launch<2, 4>(x, packed, scales, zeros, y, N, K, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_dot2(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M == 1) return gemv_rows_launch<1>(x, packed, scales, zeros, y, N, K, st);
  if (M == 2) return gemv_rows_launch<2>(x, packed, scales, zeros, y, N, K, st);
  return hipErrorInvalidValue;
}

// xs[m][k] = fp16(fp32(x[m][k]) / s[k]): one IEEE fp32 division (correctly
// rounded), then rounded once more to fp16; 8 channels per thread (K % 8 == 0).
__global__ void scale_input_kernel(const f16* __restrict__ x, const float* __restrict__ s, int64_t M, int64_t K,
                                   f16* __restrict__ xs) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // chunk of 8 channels
  if (i >= M * (K / 8)) return;
  const int64_t k0 = (i % (K / 8)) * 8;
  const uint4 v = reinterpret_cast<const uint4*>(x)[i];
  const float4 a = *reinterpret_cast<const float4*>(s + k0), b = *reinterpret_cast<const float4*>(s + k0 + 4);
  auto div_pair = [](uint32_t xw, float sa, float sb) {
    const f16x2 h = as_f16x2(xw);
    return as_u32(f16x2{(f16)((float)h.x / sa), (f16)((float)h.y / sb)});
  };
  const uint4 r{div_pair(v.x, a.x, a.y), div_pair(v.y, a.z, a.w), div_pair(v.z, b.x, b.y), div_pair(v.w, b.z, b.w)};
  reinterpret_cast<uint4*>(xs)[i] = r;
}

hipError_t launch_scale_input(const void* x, const float* s, int64_t M, int64_t K, void* xs, hipStream_t st) {
  const int64_t chunks = M * (K / 8);
  scale_input_kernel<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st>>>(
      reinterpret_cast<const f16*>(x), s, M, K, reinterpret_cast<f16*>(xs));
  return hipGetLastError();
}

}  // namespace awq
