// Measurement kernels declared in include/awq_ceilings.h: a streaming read
// with the decode GEMV's 16-byte non-temporal loads (alone, and ending each
// block with one dependent store), and a dense fp16 matrix-core loop.  They bound the libawq kernels from above on the device
// they run on; they are not part of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "awq_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One round trip per thread: each lane issues its L 16-byte pieces (the
// lanes of a block covering 256 L consecutive pieces) before using any, and
// the grid covers the whole range, so every load of the kernel is in flight
// at once up to what the device holds.  The folded value is stored only when
// it equals a fixed pattern (practically never): the kernel costs its loads
// alone, and they stay live.
template <int L>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * L + threadIdx.x;
  u32x4 v[L];
#pragma unroll
  for (int u = 0; u < L; ++u) {
    int64_t i = base + (int64_t)u * 256;
    i = i < n16 ? i : n16 - 1;
    v[u] = __builtin_nontemporal_load(src + i);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < L; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023u] = acc;
}

// The same read, finished as a decode GEMV block finishes: the block's 256
// folded words are combined (across each wave by shuffles, across the four
// waves through LDS after a barrier) and thread 0 stores the block's word to
// out[block].  Every block thus ends with one store that depends on all of its
// loads, as a GEMV block ends with its y values.
template <int L>
__global__ __launch_bounds__(256) void stream_read_store_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                uint32_t* __restrict__ out) {
  __shared__ uint32_t part[4];
  const int64_t base = (int64_t)blockIdx.x * 256 * L + threadIdx.x;
  u32x4 v[L];
#pragma unroll
  for (int u = 0; u < L; ++u) {
    int64_t i = base + (int64_t)u * 256;
    i = i < n16 ? i : n16 - 1;
    v[u] = __builtin_nontemporal_load(src + i);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < L; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Eight independent accumulation chains per wave keep the matrix core's
// pipeline full; the operands depend on the lane so nothing is constant-folded.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void mfma_f16_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(1.0f + 0.001f * (float)(lane + i));
    b[i] = (_Float16)(0.5f - 0.001f * (float)(lane - i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[c][r];
  if (lane == 0) sink[(int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6)] = t;
}

}  // namespace

extern "C" {

int awq_ceiling_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t loads_per_thread,
                            void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16) return 1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) & 15u) return 1;
  const int L = loads_per_thread;
  const int64_t n16 = (int64_t)(bytes / 16), blocks = (n16 + 256 * L - 1) / (256 * (int64_t)L);
  if (blocks >= ((int64_t)1 << 31)) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const auto p = reinterpret_cast<const u32x4*>(src);
  if (L == 1) stream_read_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n16, sink);
  else if (L == 2) stream_read_kernel<2><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n16, sink);
  else if (L == 4) stream_read_kernel<4><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n16, sink);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int awq_ceiling_stream_read_store(const void* src, size_t bytes, uint32_t* out, size_t out_words,
                                  int32_t loads_per_thread, void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16) return 1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(out)) & 15u) return 1;
  const int L = loads_per_thread;
  if (L != 1 && L != 2 && L != 4) return 1;
  const int64_t n16 = (int64_t)(bytes / 16), blocks = (n16 + 256 * L - 1) / (256 * (int64_t)L);
  if (blocks >= ((int64_t)1 << 31) || (size_t)blocks > out_words) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const auto p = reinterpret_cast<const u32x4*>(src);
  if (L == 1) stream_read_store_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n16, out);
  else if (L == 2) stream_read_store_kernel<2><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n16, out);
  else stream_read_store_kernel<4><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n16, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int awq_ceiling_mfma_f16(float* sink, int32_t blocks, int32_t iters, int32_t waves_per_simd, void* stream) {
  if (!sink || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20)) return 1;
  if (waves_per_simd != 1 && waves_per_simd != 2) return 1;
  if (reinterpret_cast<uintptr_t>(sink) & 15u) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (waves_per_simd == 1) mfma_f16_kernel<4><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(sink, iters);
  else mfma_f16_kernel<8><<<dim3((unsigned)blocks), dim3(512), 0, st>>>(sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
