// W4A16 product for M <= 16 activation rows (decode): y[m][n] = sum_k x[m][k] * w_hat[n][k].
//
// Decoding reads every weight once per token and does little arithmetic with
// it, so this kernel is bound by HBM bandwidth; 4-bit codes cut that traffic
// about 4x ("AWQ: Activation-aware Weight Quantization for On-Device LLM
// Compression and Acceleration", fdeinterviews.com/papers/awq, paragraphs 1
// and 6).  Codes are dequantized on the fly in registers (OpenAlex record of
// the GetMobile AWQ article, abstract).
//
// Design for gfx950: the dot products run on the matrix cores
// (v_mfma_f32_16x16x32_f16) with the activations as the A operand (rows m,
// zero beyond M) and the weights as the B operand.  The B operand of one lane
// is 8 consecutive input channels of one weight row -- exactly one packed
// word -- so a lane unpacks its word in registers: one shift and one and-or
// per channel pair give fp16 1024 + code (the packed nibble order puts
// channels 2j and 2j+1 in the two halves of (word >> 4j) & 0x000F000F) and one
// packed fp16 subtraction of 1024 + zero gives (code - zero) exactly.  The
// matrix core accumulates a 128-channel group in fp32; the group's fp16 scale
// is then applied in fp32.  No cross-lane reduction is needed, and the vector
// ALU work per weight does not grow with M.
//
// Mapping: a block owns 16*RW weight rows and all of K; its W waves split the
// K groups (wave w takes groups w, w+W, ...).  For one group a wave loads 16 B
// per lane: lane l reads the (l/16)-th 16-byte quarter of the group's 64 B in
// row l%16, so one load instruction fetches 16 rows x 64 B.  All loads of a
// batch of P groups (and, without LDS staging, their x fragments) are issued
// before any is used.  x is staged once per block in LDS when it fits, before
// the first weight load.  The waves' partial tiles are summed through LDS
// in a fixed order, so results are deterministic.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kSkinnyMaxWaves = 8;
constexpr size_t kSkinnyLdsBudget = 64 * 1024;

// Waves per block: about P groups per wave, at most kSkinnyMaxWaves.  It is a
// function of K alone, so the kernel derives it from its arguments (which the
// hardware preloads into registers) instead of reading the dispatch packet.
template <int P>
__host__ __device__ inline int skinny_waves(int64_t K) {
  const int64_t w = (K / kGroup + P - 1) / P;
  return w < 1 ? 1 : (w > kSkinnyMaxWaves ? kSkinnyMaxWaves : (int)w);
}

template <int RW, int P, int MT, bool XLDS>
__global__ __launch_bounds__(512) void skinny_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                     const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                     f16* __restrict__ y, int M, int N32, int K32, int red_offset) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int64_t N = N32, K = K32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W = skinny_waves<P>(K);  // == blockDim.x / 64
  const int nl = lane & 15, kq = lane >> 4;  // row within a 16-row tile; quarter of a group
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RW);
  const int64_t K8 = K / 8, G = K / kGroup, P2 = (G + 1) / 2;
  // A-operand rows past M read row M - 1 (valid memory): MFMA output rows are
  // independent and those rows are never stored.
  int64_t xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xrow[mt] = 16 * mt + nl < M ? 16 * mt + nl : M - 1;

  int64_t rowi[RW];
#pragma unroll
  for (int t = 0; t < RW; ++t) {
    const int64_t n = n0 + 16 * t + nl;
    rowi[t] = n < N ? n : N - 1;  // tail rows reload the last row; never stored
  }
  f32x4 acc[RW][MT];
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // x goes into LDS before any weight load is issued: vector-memory loads
  // complete in order, so waiting for the copy must not include them.
  f16* xs = reinterpret_cast<f16*>(smem);
  if (XLDS) {
    const int64_t n16 = (int64_t)M * K / 8;
    for (int64_t i = threadIdx.x; i < n16; i += W * kWave)
      reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
    __syncthreads();
  }
  // Without LDS staging the batch's x fragments are loaded together with its
  // weights, before the first wait, when they fit in registers; otherwise per group.
  constexpr bool XPRE = !XLDS && P * MT <= 4;

  for (int64_t gb = wave; gb < G; gb += (int64_t)W * P) {
    u32x4 wv[P][RW];
    f16 sc[P][RW];
    uint32_t zz[P][RW];
    f16x8 ap[XPRE ? P : 1][MT][4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t g = gb + (int64_t)p * W;
      const int64_t gg = g < G ? g : G - 1;  // past the last group: reloaded, never used
      if constexpr (XPRE) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            ap[p][mt][s] = *reinterpret_cast<const f16x8*>(x + xrow[mt] * K + gg * kGroup + kq * 32 + 8 * s);
      }
#pragma unroll
      for (int t = 0; t < RW; ++t) {
        wv[p][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(packed + rowi[t] * K8 + gg * 16 + kq * 4));
        sc[p][t] = scales[rowi[t] * G + gg];
        zz[p][t] = (zeros[rowi[t] * P2 + (gg >> 1)] >> (4 * (gg & 1))) & 0xFu;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch before the first wait
#pragma unroll
    for (int p = 0; p < P; ++p) {
      // branch-free: a group past the last one recomputes the last and adds 0
      // (a branch here would let the compiler sink this group's loads below
      // the previous group's wait)
      const int64_t g = gb + (int64_t)p * W;
      const bool live = g < G;
      const int64_t k0 = (live ? g : G - 1) * kGroup + kq * 32;
      f16x8 a[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (XPRE) a[mt][s] = ap[p][mt][s];
          else if constexpr (XLDS) a[mt][s] = *reinterpret_cast<const f16x8*>(xs + xrow[mt] * K + k0 + 8 * s);
          else a[mt][s] = *reinterpret_cast<const f16x8*>(x + xrow[mt] * K + k0 + 8 * s);
        }
#pragma unroll
      for (int t = 0; t < RW; ++t) {
        const f16x2 zb = zero_biased(zz[p][t]);
        f32x4 d[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) d[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t word = wv[p][t][s];
          const f16x2 q0 = pair_biased(word, 0) - zb, q1 = pair_biased(word, 1) - zb;
          const f16x2 q2 = pair_biased(word, 2) - zb, q3 = pair_biased(word, 3) - zb;
          const f16x8 b = f16x8{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][s], b, d[mt], 0, 0, 0);
        }
        const float scf = live ? (float)sc[p][t] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][mt][r] = fmaf(scf, d[mt][r], acc[t][mt][r]);
      }
    }
  }

  // sum the waves' tiles: lane holds y[m = 16*mt + 4*kq + r][n0 + 16t + nl]
  float* red = reinterpret_cast<float*>(smem + red_offset);
  if (MT == 1) {  // one slot per wave, then a fixed-order sum per output
#pragma unroll
    for (int t = 0; t < RW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m < M) red[((wave * RW + t) * 16 + m) * 16 + nl] = acc[t][0][r];
      }
    __syncthreads();
    for (int i = threadIdx.x; i < RW * 16 * M; i += W * kWave) {
      const int t = i / (16 * M), rem = i - t * 16 * M, m = rem >> 4, nn = rem & 15;
      float v = 0.f;
      for (int w = 0; w < W; ++w) v += red[((w * RW + t) * 16 + m) * 16 + nn];
      const int64_t n = n0 + 16 * t + nn;
      if (n < N) y[(int64_t)m * N + n] = (f16)v;
    }
  } else {  // one tile, accumulated wave by wave in a fixed order
    constexpr int MR = 16 * MT;
    for (int w = 0; w < W; ++w) {
      if (wave == w) {
#pragma unroll
        for (int t = 0; t < RW; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = 16 * mt + 4 * kq + r;
              float& dst = red[(t * MR + m) * 16 + nl];
              dst = (w == 0 ? 0.f : dst) + acc[t][mt][r];
            }
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < RW * 16 * M; i += W * kWave) {
      const int t = i / (16 * M), rem = i - t * 16 * M, m = rem >> 4, nn = rem & 15;
      const int64_t n = n0 + 16 * t + nn;
      if (n < N) y[(int64_t)m * N + n] = (f16)red[(t * MR + m) * 16 + nn];
    }
  }
}

template <int RW, int P, int MT = 1>
static hipError_t skinny_launch(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                                int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int W = skinny_waves<P>(K);
  const size_t red_bytes = (size_t)(MT == 1 ? W : 1) * RW * 16 * MT * 16 * sizeof(float);
  const size_t xbytes = (size_t)M * (size_t)K * 2;
  const bool xlds = xbytes + red_bytes <= kSkinnyLdsBudget;
  const size_t red_offset = xlds ? xbytes : 0;
  const size_t lds = red_offset + red_bytes;
  dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW))), block((unsigned)(W * kWave));
  auto xp = reinterpret_cast<const f16*>(x);
  auto pp = reinterpret_cast<const uint32_t*>(packed);
  auto sp = reinterpret_cast<const f16*>(scales);
  auto zp = reinterpret_cast<const uint8_t*>(zeros);
  auto yp = reinterpret_cast<f16*>(y);
  if (xlds)
    skinny_kernel<RW, P, MT, true><<<grid, block, lds, st>>>(xp, pp, sp, zp, yp, (int)M, (int)N, (int)K, (int)red_offset);
  else
    skinny_kernel<RW, P, MT, false><<<grid, block, lds, st>>>(xp, pp, sp, zp, yp, (int)M, (int)N, (int)K, (int)red_offset);
  return hipGetLastError();
}

// 17 <= M <= 64: the same kernel with M in up to four 16-row m-tiles; each
// unpacked weight operand feeds one MFMA per m-tile.  Measured against the
// pipelined GEMM (M = 17, 32, 48, 64 on the 7B/70B shapes) it wins on layers
// up to 8192 wide (two tiles per wave: 4096 x 4096 at 15-27 us against 32 us,
// 11008 x 4096 at 34-60 us against 72 us) and, with four tiles per wave in
// batches of two groups, on wider K = 4096 layers up to M = 48 (4096 x 11008
// at 22-30 us against 33 us); elsewhere the GEMM is faster.
bool gemv_wide_preferred(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || M > 64) return false;
  return N <= 8192 || (M <= 48 && K <= 4096);
}

template <int RW, int P>
static hipError_t wide_launch(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                              int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 32) return skinny_launch<RW, P, 2>(x, packed, scales, zeros, y, M, N, K, st);
  if (M <= 48) return skinny_launch<RW, P, 3>(x, packed, scales, zeros, y, M, N, K, st);
  return skinny_launch<RW, P, 4>(x, packed, scales, zeros, y, M, N, K, st);
}

hipError_t launch_gemv_wide(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 16 || M > 64) return hipErrorInvalidValue;
  if (N <= 8192) return wide_launch<2, 1>(x, packed, scales, zeros, y, M, N, K, st);
  return wide_launch<4, 2>(x, packed, scales, zeros, y, M, N, K, st);
}

// Tile shape, measured on the Llama-2 7B/70B decode shapes at M = 4, 8, 16:
// one 16-row tile per wave by default; on wide layers (N >= 16384, or
// N >= 8192 with K = 4096 and M > 8) four tiles per wave in batches of two
// groups share each x fragment over more weight rows (8192 x 28672: 59-68 us
// against 74-81 us; 4096 x 11008 at M = 16: 18 us against 21 us); on long K
// (>= 16384), and for M > 8 on 8192-wide layers with K >= 8192, two tiles per
// wave, which still leaves at least 256 blocks (8192 x 8192 at M = 16: 24 us
// against 37 us with four tiles).
hipError_t launch_gemv(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t st) {
  if (M < 1 || M > 16) return hipErrorInvalidValue;
  if (gemv_dot2_supported(M, K)) return launch_gemv_dot2(x, packed, scales, zeros, y, M, N, K, st);
  if (K >= 16384) return skinny_launch<2, 4>(x, packed, scales, zeros, y, M, N, K, st);
  if (N >= 16384 || (M > 8 && N >= 8192 && K <= 4096)) return skinny_launch<4, 2>(x, packed, scales, zeros, y, M, N, K, st);
  if (M > 8 && N >= 8192) return skinny_launch<2, 4>(x, packed, scales, zeros, y, M, N, K, st);
  return skinny_launch<1, 4>(x, packed, scales, zeros, y, M, N, K, st);
}

}  // namespace awq
