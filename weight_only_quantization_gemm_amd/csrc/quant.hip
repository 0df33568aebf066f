// Per-channel scales s = a^alpha, the group-wise int4 / int3 quantizer, the
// weight error used by the search loss, and the packers.
//
// Method: a weight channel is multiplied by s and its input divided by s,
// which leaves the layer's output unchanged in exact arithmetic while the
// channel's rounding error shrinks relative to its size; s is the channel's
// average activation magnitude raised to alpha ("AWQ: Activation-aware Weight
// Quantization for On-Device LLM Compression and Acceleration",
// fdeinterviews.com/papers/awq, paragraph 3).  The group quantizer (group 128,
// min-max asymmetric, fp16 step, integer zero point, round-half-even) is this
// library's reading of the 4-bit weight-only format the pages name; the pages
// also evaluate 3-bit weights (same page, paragraphs 4 and 10), which take the
// same quantizer with 8 levels instead of 16.
//
// Every float operation below is an IEEE fp32/fp64 operation rounded to
// nearest-even (the file is built with -ffp-contract=off and correctly
// rounded division), so codes, zero points and steps are reproducible
// bit-for-bit by any implementation that performs the same operations.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

// s_all[i][k] = fp32(a_k ^ alpha_i) (1 where a_k = 0), and inv_all[i][k] =
// 1 / s in fp64 for the error kernels (one division per channel and alpha
// here instead of one per weight there).
__global__ void scales_kernel(const double* __restrict__ a, AlphaGrid al, int n_alpha, int64_t K,
                              float* __restrict__ s_all, double* __restrict__ inv_all) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int i = blockIdx.y;
  if (k >= K || i >= n_alpha) return;
  double ak = a[k];
  float s = (ak == 0.0) ? 1.0f : (float)pow(ak, (double)al.v[i]);
  s_all[(int64_t)i * K + k] = s;
  inv_all[(int64_t)i * K + k] = 1.0 / (double)s;
}

hipError_t launch_scales(const double* a, const AlphaGrid& al, int n_alpha, int64_t K, float* s_all,
                         double* inv_all, hipStream_t st) {
  dim3 grid((unsigned)((K + 255) / 256), (unsigned)n_alpha);
  scales_kernel<<<grid, dim3(256), 0, st>>>(a, al, n_alpha, K, s_all, inv_all);
  return hipGetLastError();
}

// Quantizes the 8 consecutive weights one thread holds; the 16 threads of an
// aligned 16-lane segment hold one 128-channel group and agree on its range.
struct Quant8 {
  float v[8];   // scaled weights
  float q[8];   // codes
  float z;      // zero point
  float sc;     // fp16 step as float
  f16 sc16;
};

__device__ inline void unpack_w8(const uint4 raw, float w[8]) {
  const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h = as_f16x2(r[i]);
    w[2 * i] = (float)h.x;
    w[2 * i + 1] = (float)h.y;
  }
}

__device__ inline void load_w8(const uint4* W, int64_t idx, float w[8]) { unpack_w8(W[idx], w); }

__device__ inline void load_s8(const float* s, int64_t k0, float out[8]) {
  if (s == nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 1.0f;
    return;
  }
  float4 a = *reinterpret_cast<const float4*>(s + k0);
  float4 b = *reinterpret_cast<const float4*>(s + k0 + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

template <int QMAX>
__device__ inline void quantize8(const float w[8], const float s[8], Quant8& r) {
  float mn = 0.0f, mx = 0.0f;  // the range always contains 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r.v[i] = w[i] * s[i];
    mn = fminf(mn, r.v[i]);
    mx = fmaxf(mx, r.v[i]);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 16));
    mx = fmaxf(mx, __shfl_xor(mx, off, 16));
  }
  constexpr float qmax = (float)QMAX;
  float step = (mx - mn) / qmax;
  step = fmaxf(step, 0x1p-14f);
  r.sc16 = (f16)step;
  r.sc = (float)r.sc16;
  r.z = fminf(fmaxf(rintf(-mn / r.sc), 0.0f), qmax);
#pragma unroll
  for (int i = 0; i < 8; ++i) r.q[i] = fminf(fmaxf(rintf(r.v[i] / r.sc) + r.z, 0.0f), qmax);
}

// The fp64 factors 1/s of 8 channels (1 where s is NULL).
__device__ inline void load_inv8(const double* inv, int64_t k0, double out[8]) {
  if (inv == nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 1.0;
    return;
  }
  const double2* p = reinterpret_cast<const double2*>(inv + k0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double2 v = p[i];
    out[2 * i] = v.x;
    out[2 * i + 1] = v.y;
  }
}

// E = w_hat / s - w in fp64 as one fma of the exact w_hat = (q - z) * sc (an
// integer times an fp16 value, exact in fp32) with the fp64 1/s: within one
// fp64 rounding of the quotient form, far below the fp32 E is kept in.
__device__ inline double weight_error(float q, float z, float sc, double inv, float w) {
  return fma((double)((q - z) * sc), inv, -(double)w);
}

// Rows per thread of the error kernels: a thread keeps its 8 channels' s, 1/s
// and exponents in registers for kErrRows rows of W, whose words it loads
// together before quantizing them.
constexpr int kErrRows = 8;

// Weight error of the search, pre-scaled for the loss contraction:
// E'[n][k] = (w_hat / s - w) * 2^e_k, evaluated in fp64, rounded to fp32 and
// stored as an fp16 pair hi = fp16(E'), lo = fp16(E' - hi).  Thread (row block
// rb, word w) takes channels 8w .. 8w + 7 of rows kErrRows rb .. + kErrRows - 1;
// the 16 threads of an aligned segment hold one 128-channel group of the same
// rows (K / 8 is a multiple of 16).  Channels with keep[k] != 0 (keep may be
// NULL) stay exact: their error is 0.
template <int QMAX>
__global__ __launch_bounds__(256) void quant_error_kernel(const uint4* __restrict__ W, const float* __restrict__ s,
                                                          const double* __restrict__ inv,
                                                          const int32_t* __restrict__ ex,
                                                          const uint8_t* __restrict__ keep, int64_t N, int64_t K,
                                                          f16* __restrict__ Ehi, f16* __restrict__ Elo) {
  const int64_t K8 = K / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rb = idx / K8, w = idx - rb * K8, n0 = rb * kErrRows;
  // the grid covers whole 16-lane segments, and all lanes of a segment share rb
  if (n0 >= N) return;
  float sf[8];
  double iv[8];
  int32_t e8[8];
  bool kept[8];
  load_s8(s, w * 8, sf);
  load_inv8(inv, w * 8, iv);
  {
    const int4 a = *reinterpret_cast<const int4*>(ex + w * 8), b = *reinterpret_cast<const int4*>(ex + w * 8 + 4);
    e8[0] = a.x; e8[1] = a.y; e8[2] = a.z; e8[3] = a.w;
    e8[4] = b.x; e8[5] = b.y; e8[6] = b.z; e8[7] = b.w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) kept[i] = keep != nullptr && keep[w * 8 + i];
  uint4 raw[kErrRows];
#pragma unroll
  for (int r = 0; r < kErrRows; ++r) raw[r] = W[(n0 + r < N ? n0 + r : N - 1) * K8 + w];
#pragma unroll
  for (int r = 0; r < kErrRows; ++r) {
    const int64_t n = n0 + r;
    if (n >= N) break;  // uniform over the segment
    float wf[8];
    unpack_w8(raw[r], wf);
    Quant8 q;
    quantize8<QMAX>(wf, sf, q);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      f16x2 h, l;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        double e = weight_error(q.q[i + u], q.z, q.sc, iv[i + u], wf[i + u]);
        if (kept[i + u]) e = 0.0;
        const float v = (float)ldexp(e, e8[i + u]);
        const f16 hi = (f16)v;
        h[u] = hi;
        l[u] = (f16)(v - (float)hi);
      }
      hw[i / 2] = as_u32(h);
      lw[i / 2] = as_u32(l);
    }
    *reinterpret_cast<uint4*>(Ehi + n * K + w * 8) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(Elo + n * K + w * 8) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// Unscaled weight error in fp32 for the direct form of the loss; the same
// mapping as above.
template <int QMAX>
__global__ __launch_bounds__(256) void quant_error32_kernel(const uint4* __restrict__ W, const float* __restrict__ s,
                                                            const double* __restrict__ inv,
                                                            const uint8_t* __restrict__ keep, int64_t N, int64_t K,
                                                            float* __restrict__ E) {
  const int64_t K8 = K / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rb = idx / K8, w = idx - rb * K8, n0 = rb * kErrRows;
  if (n0 >= N) return;  // whole 16-lane segments, as above
  float sf[8];
  double iv[8];
  bool kept[8];
  load_s8(s, w * 8, sf);
  load_inv8(inv, w * 8, iv);
#pragma unroll
  for (int i = 0; i < 8; ++i) kept[i] = keep != nullptr && keep[w * 8 + i];
  uint4 raw[kErrRows];
#pragma unroll
  for (int r = 0; r < kErrRows; ++r) raw[r] = W[(n0 + r < N ? n0 + r : N - 1) * K8 + w];
#pragma unroll
  for (int r = 0; r < kErrRows; ++r) {
    const int64_t n = n0 + r;
    if (n >= N) break;
    float wf[8];
    unpack_w8(raw[r], wf);
    Quant8 q;
    quantize8<QMAX>(wf, sf, q);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = kept[i] ? 0.0f : (float)weight_error(q.q[i], q.z, q.sc, iv[i], wf[i]);
    float4* out = reinterpret_cast<float4*>(E + n * K + w * 8);
    out[0] = make_float4(e[0], e[1], e[2], e[3]);
    out[1] = make_float4(e[4], e[5], e[6], e[7]);
  }
}

static dim3 error_grid(int64_t N, int64_t K) {
  const int64_t threads = (N + kErrRows - 1) / kErrRows * (K / 8);
  return dim3((unsigned)((threads + 255) / 256));
}

hipError_t launch_quant_error32(const void* W, const float* s, const double* inv, const uint8_t* keep, int64_t N,
                                int64_t K, int bits, float* E, hipStream_t st) {
  const dim3 grid = error_grid(N, K), block(256);
  auto Wp = reinterpret_cast<const uint4*>(W);
  if (bits == 3) quant_error32_kernel<7><<<grid, block, 0, st>>>(Wp, s, inv, keep, N, K, E);
  else quant_error32_kernel<15><<<grid, block, 0, st>>>(Wp, s, inv, keep, N, K, E);
  return hipGetLastError();
}

hipError_t launch_quant_error(const void* W, const float* s, const double* inv, const int32_t* ex,
                              const uint8_t* keep, int64_t N, int64_t K, int bits, void* Ehi, void* Elo,
                              hipStream_t st) {
  const dim3 grid = error_grid(N, K), block(256);
  auto Wp = reinterpret_cast<const uint4*>(W);
  auto hi = reinterpret_cast<f16*>(Ehi);
  auto lo = reinterpret_cast<f16*>(Elo);
  if (bits == 3) quant_error_kernel<7><<<grid, block, 0, st>>>(Wp, s, inv, ex, keep, N, K, hi, lo);
  else quant_error_kernel<15><<<grid, block, 0, st>>>(Wp, s, inv, ex, keep, N, K, hi, lo);
  return hipGetLastError();
}

// Top channels: out[r] = k for the channel k of rank r < n_keep, the rank being
// the number of channels with a larger value plus those with an equal value
// and a lower index (largest first, ties to the lower index).  Every value is
// compared exactly, so the choice is reproducible bit for bit.
__global__ __launch_bounds__(256) void top_channels_kernel(const double* __restrict__ v, int K, int n_keep,
                                                           int32_t* __restrict__ out) {
  __shared__ double tile[256];
  const int k = blockIdx.x * 256 + threadIdx.x;
  const double vk = k < K ? v[k] : 0.0;
  int rank = 0;
  for (int j0 = 0; j0 < K; j0 += 256) {
    __syncthreads();
    if (j0 + (int)threadIdx.x < K) tile[threadIdx.x] = v[j0 + threadIdx.x];
    __syncthreads();
    const int jn = K - j0 < 256 ? K - j0 : 256;
    for (int j = 0; j < jn; ++j) {
      const double vj = tile[j];
      rank += (vj > vk) || (vj == vk && j0 + j < k);
    }
  }
  if (k < K && rank < n_keep) out[rank] = k;
}

hipError_t launch_top_channels(const double* v, int64_t K, int n_keep, int32_t* out, hipStream_t st) {
  top_channels_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(v, (int)K, n_keep, out);
  return hipGetLastError();
}

__global__ void keep_mask_clear_kernel(uint8_t* __restrict__ mask, int64_t K) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < K) mask[k] = 0;
}

__global__ void keep_mask_set_kernel(const int32_t* __restrict__ keep, int n_keep, int64_t K,
                                     uint8_t* __restrict__ mask) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_keep) {
    const int32_t k = keep[i];
    if (k >= 0 && k < K) mask[k] = 1;  // out-of-range entries are ignored
  }
}

hipError_t launch_keep_mask(const int32_t* keep, int n_keep, int64_t K, uint8_t* mask, hipStream_t st) {
  keep_mask_clear_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(mask, K);
  if (n_keep > 0)
    keep_mask_set_kernel<<<dim3((unsigned)((n_keep + 255) / 256)), dim3(256), 0, st>>>(keep, n_keep, K, mask);
  return hipGetLastError();
}

// Packers: a 32-lane segment handles the group pair (2p, 2p+1) of one row so
// that the two zero points of a zeros byte are known to one lane; lane i of a
// 16-lane half quantizes channels 8i .. 8i + 7 of its group.
//
// 4-bit words: the code of channel 8w + i of a row sits in nibble
// 4 (i % 2) + i / 2 of word w.  3-bit: the 32 channels 32c .. 32c + 31 of a
// row are the three words 3c .. 3c + 2; the code of channel 2p (p = 0..14)
// sits in bits 3j .. 3j + 2 of word p / 5 (j = p % 5), that of channel 2p + 1
// in bits 16 + 3j .. 16 + 3j + 2 of the same word, and bit b of the codes of
// channels 30 and 31 in bits 15 and 31 of word b.  A chunk of 32 channels is
// four lanes' codes, OR-ed together across the four lanes.
template <int BITS>
__device__ inline void pack3_bits(const float q[8], int sub, uint32_t w[3]) {
  w[0] = w[1] = w[2] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = (uint32_t)q[i];
    const int ch = 8 * sub + i;  // channel within the 32-channel chunk
    if (ch < 30) {
      const int p = ch >> 1, t = p / 5, j = p - 5 * t;
      const uint32_t bits = code << (3 * j + 16 * (ch & 1));
      w[0] |= t == 0 ? bits : 0u;
      w[1] |= t == 1 ? bits : 0u;
      w[2] |= t == 2 ? bits : 0u;
    } else {
      const int at = ch == 30 ? 15 : 31;
#pragma unroll
      for (int b = 0; b < 3; ++b) w[b] |= ((code >> b) & 1u) << at;
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ W, const float* __restrict__ s,
                                                   int64_t N, int64_t K, uint32_t* __restrict__ packed,
                                                   f16* __restrict__ scales, uint8_t* __restrict__ zeros) {
  const int64_t G = K / kGroup;
  const int64_t P = (G + 1) / 2;  // group pairs per row == zeros bytes per row
  const int64_t seg = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
  const int lane32 = threadIdx.x & 31;
  if (seg >= N * P) return;  // whole 32-lane segments exit together
  const int64_t n = seg / P, p = seg - n * P;
  const int64_t g = 2 * p + (lane32 >> 4);
  const bool live = g < G;
  const int64_t w = g * 16 + (lane32 & 15);  // 8-channel word within the row
  float wf[8], sf[8];
  if (live) {
    load_w8(W, n * (K / 8) + w, wf);
    load_s8(s, w * 8, sf);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) { wf[i] = 0.0f; sf[i] = 1.0f; }
  }
  Quant8 r;
  quantize8<(1 << BITS) - 1>(wf, sf, r);  // a dead half-segment quantizes zeros and is discarded
  uint32_t z_other = (uint32_t)__shfl_xor((int)r.z, 16, 32);
  if constexpr (BITS == 4) {
    if (!live) return;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= ((uint32_t)r.q[i]) << (4 * nibble_pos(i));
    packed[n * (K / 8) + w] = word;
  } else {
    uint32_t cw[3];
    pack3_bits<BITS>(r.q, lane32 & 3, cw);
#pragma unroll
    for (int b = 0; b < 3; ++b) {  // OR over the chunk's four lanes (all lanes take part)
      cw[b] |= (uint32_t)__shfl_xor((int)cw[b], 1, 32);
      cw[b] |= (uint32_t)__shfl_xor((int)cw[b], 2, 32);
    }
    if (!live) return;
    if ((lane32 & 3) == 0) {
      uint32_t* dst = packed + (n * (K / 32) + (w >> 2)) * 3;
      dst[0] = cw[0];
      dst[1] = cw[1];
      dst[2] = cw[2];
    }
  }
  if ((lane32 & 15) == 0) scales[n * G + g] = r.sc16;
  if (lane32 == 0) {
    uint32_t zlo = (uint32_t)r.z;
    uint32_t zhi = (g + 1 < G) ? z_other : 0u;
    zeros[n * P + p] = (uint8_t)(zlo | (zhi << 4));
  }
}

hipError_t launch_pack(const void* W, const float* s, int64_t N, int64_t K, int bits, void* packed, void* scales,
                       void* zeros, hipStream_t st) {
  const int64_t G = K / kGroup, P = (G + 1) / 2;
  const int64_t threads = N * P * 32;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  auto Wp = reinterpret_cast<const uint4*>(W);
  auto pp = reinterpret_cast<uint32_t*>(packed);
  auto sp = reinterpret_cast<f16*>(scales);
  auto zp = reinterpret_cast<uint8_t*>(zeros);
  if (bits == 3) pack_kernel<3><<<grid, block, 0, st>>>(Wp, s, N, K, pp, sp, zp);
  else pack_kernel<4><<<grid, block, 0, st>>>(Wp, s, N, K, pp, sp, zp);
  return hipGetLastError();
}

__global__ void select_scale_kernel(const float* __restrict__ s_all, const int32_t* __restrict__ best, int64_t K,
                                    float* __restrict__ s_out) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < K) s_out[k] = s_all[(int64_t)best[0] * K + k];
}

hipError_t launch_select_scale(const float* s_all, const int32_t* best, int64_t K, float* s_out, hipStream_t st) {
  select_scale_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(s_all, best, K, s_out);
  return hipGetLastError();
}

__global__ void unpack_kernel(const uint32_t* __restrict__ packed, const uint8_t* __restrict__ zeros, int64_t N,
                              int64_t K, uint8_t* __restrict__ codes, uint8_t* __restrict__ zeros_u8) {
  const int64_t K8 = K / 8, G = K / kGroup, P = (G + 1) / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * K8) return;
  const int64_t n = idx / K8, w = idx - n * K8;
  const uint32_t word = packed[idx];
#pragma unroll
  for (int i = 0; i < 8; ++i) codes[n * K + w * 8 + i] = (uint8_t)((word >> (4 * nibble_pos(i))) & 0xFu);
  if ((w & 15) == 0) {
    const int64_t g = w >> 4;
    zeros_u8[n * G + g] = (uint8_t)((zeros[n * P + (g >> 1)] >> (4 * (g & 1))) & 0xFu);
  }
}

// One thread per 32-channel chunk of the 3-bit format.
__global__ void unpack3_kernel(const uint32_t* __restrict__ packed, const uint8_t* __restrict__ zeros, int64_t N,
                               int64_t K, uint8_t* __restrict__ codes, uint8_t* __restrict__ zeros_u8) {
  const int64_t K32 = K / 32, G = K / kGroup, P = (G + 1) / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * K32) return;
  const int64_t n = idx / K32, c = idx - n * K32;
  const uint32_t w[3] = {packed[3 * idx], packed[3 * idx + 1], packed[3 * idx + 2]};
  uint8_t* out = codes + n * K + c * 32;
#pragma unroll
  for (int p = 0; p < 15; ++p) {
    const uint32_t v = w[p / 5] >> (3 * (p % 5));
    out[2 * p] = (uint8_t)(v & 7u);
    out[2 * p + 1] = (uint8_t)((v >> 16) & 7u);
  }
  out[30] = (uint8_t)(((w[0] >> 15) & 1u) | (((w[1] >> 15) & 1u) << 1) | (((w[2] >> 15) & 1u) << 2));
  out[31] = (uint8_t)(((w[0] >> 31) & 1u) | (((w[1] >> 31) & 1u) << 1) | (((w[2] >> 31) & 1u) << 2));
  if ((c & 3) == 0) {
    const int64_t g = c >> 2;
    zeros_u8[n * G + g] = (uint8_t)((zeros[n * P + (g >> 1)] >> (4 * (g & 1))) & 0xFu);
  }
}

hipError_t launch_unpack(const void* packed, const void* zeros, int64_t N, int64_t K, int bits, uint8_t* codes,
                         uint8_t* zeros_u8, hipStream_t st) {
  auto pp = reinterpret_cast<const uint32_t*>(packed);
  auto zp = reinterpret_cast<const uint8_t*>(zeros);
  if (bits == 3) {
    const int64_t chunks = N * (K / 32);
    unpack3_kernel<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st>>>(pp, zp, N, K, codes, zeros_u8);
  } else {
    const int64_t words = N * (K / 8);
    unpack_kernel<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st>>>(pp, zp, N, K, codes, zeros_u8);
  }
  return hipGetLastError();
}

}  // namespace awq
