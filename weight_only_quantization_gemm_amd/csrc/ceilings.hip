// Measurement kernels declared in include/awq_ceilings.h: a streaming read
// with the decode GEMV's 16-byte non-temporal loads, and a dense fp16
// matrix-core loop.  They bound the libawq kernels from above on the device
// they run on; they are not part of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "awq_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four 16-byte pieces per lane per round (all issued before any is used), the
// lanes of the grid covering consecutive pieces.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
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

int awq_ceiling_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || blocks < 1 || blocks > 65536) return 1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) & 15u) return 1;
  stream_read_kernel<<<dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
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
