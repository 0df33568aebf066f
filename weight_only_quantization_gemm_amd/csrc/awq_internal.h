// Host-side launchers of the libawq kernels (internal; the public interface is
// include/awq.h).  Each enqueues its kernels on `st` and returns the launch
// status; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

constexpr int kMaxAlphas = 64;

struct AlphaGrid {
  float v[kMaxAlphas];
};

// stats.hip
hipError_t launch_channel_mean_abs(const void* X, int64_t M, int64_t K, double* a, hipStream_t st);
hipError_t launch_transpose(const void* X, int64_t M, int64_t K, int64_t Mp, void* Xt, hipStream_t st);

// gram.hip: G = Xt Xt^T (fp32 [K][K], fp64 accumulation) from Xt fp16 [K][Mp], Mp % 64 == 0, K % 64 == 0.
// partial: gram_partial_bytes(K, Mp) bytes of device scratch (may be null when that is 0)
hipError_t launch_gram(const void* Xt, int64_t Mp, int64_t K, float* G, double* partial, hipStream_t st);
size_t gram_partial_bytes(int64_t K, int64_t Mp);

// quant.hip
// s_all fp32 [n_alpha][K] and inv_all = 1 / s_all in fp64
hipError_t launch_scales(const double* a, const AlphaGrid& al, int n_alpha, int64_t K, float* s_all,
                         double* inv_all, hipStream_t st);
// bits: 4 (16 levels) or 3 (8 levels); s and inv (its fp64 reciprocal) both NULL or both given
// keep: NULL, or uint8 [K] marking channels whose error is 0 (kept exact)
hipError_t launch_quant_error(const void* W, const float* s, const double* inv, const int32_t* ex,
                              const uint8_t* keep, int64_t N, int64_t K, int bits, void* Ehi, void* Elo,
                              hipStream_t st);
hipError_t launch_quant_error32(const void* W, const float* s, const double* inv, const uint8_t* keep, int64_t N,
                                int64_t K, int bits, float* E, hipStream_t st);
hipError_t launch_top_channels(const double* v, int64_t K, int n_keep, int32_t* out, hipStream_t st);
hipError_t launch_keep_mask(const int32_t* keep, int n_keep, int64_t K, uint8_t* mask, hipStream_t st);
hipError_t launch_pack(const void* W, const float* s, int64_t N, int64_t K, int bits, void* packed, void* scales,
                       void* zeros, hipStream_t st);
hipError_t launch_select_scale(const float* s_all, const int32_t* best, int64_t K, float* s_out, hipStream_t st);
hipError_t launch_unpack(const void* packed, const void* zeros, int64_t N, int64_t K, int bits, uint8_t* codes,
                         uint8_t* zeros_u8, hipStream_t st);

// loss.hip: channel exponents and the fp16 split of the scaled Gram matrix;
// partials of sum_n E'_n G' E'_n^T; reduce + argmin.
hipError_t launch_gram_split(const float* G, int64_t K, int32_t* e, void* Ghi, void* Glo, hipStream_t st);
int64_t loss_partial_count(int64_t N, int64_t K);
hipError_t launch_loss_partials(const void* Ehi, const void* Elo, const void* Ghi, const void* Glo, int64_t N,
                                int64_t K, double* partial, hipStream_t st);
int64_t loss_direct_partial_count(int64_t M, int64_t N);
hipError_t launch_loss_direct(const void* X, const float* E, int64_t M, int64_t N, int64_t K, double* partial,
                              hipStream_t st);
hipError_t launch_loss_reduce(const double* partial, int64_t count, double mn, double* loss, hipStream_t st);
hipError_t launch_argmin(const double* loss, int n, int32_t* best, hipStream_t st);

// gemv.hip (vector-ALU GEMV, M <= 2), skinny.hip (matrix-core decode kernels: LDS-ring kernel for M <= 16, register-staged up to
// 64 where it beats the GEMM), gemm.hip / gemm_pipe.hip (matrix-core GEMM)
bool gemv_dot2_supported(int64_t M, int64_t K);
// The input side of the per-channel scaling: xs = fp16(x / s).
hipError_t launch_scale_input(const void* x, const float* s, int64_t M, int64_t K, void* xs, hipStream_t st);
hipError_t launch_gemv_dot2(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t st);
bool ring3_supported(int64_t M, int64_t N, int64_t K);
bool ring_mid_supported(int64_t M, int64_t N, int64_t K, int bits);  // 17 <= M <= 64 on the ring kernel
hipError_t launch_ring_mid(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                           int64_t M, int64_t N, int64_t K, int bits, hipStream_t st);
hipError_t launch_ring3(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                        int64_t M, int64_t N, int64_t K, hipStream_t st);
bool gemv_wide_preferred(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_wide(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemv(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st);
bool gemm_pipe_supported(int64_t M, int64_t N, int64_t K);
bool gemm_pipe3_supported(int64_t M, int64_t N, int64_t K);  // 3-bit codes, M > 16
bool ring_mid_pipe_preferred(int64_t M, int64_t N, int64_t K);
// ws: null, or gemm_pipe_workspace_bytes(M, N) bytes whose counter part is zero (left zero): the
// pipelined GEMM then splits its work evenly over the compute units (stream-K)
size_t gemm_pipe_workspace_bytes(int64_t M, int64_t N);
// whether the pipelined GEMM splits its work (stream-K) when it is given a workspace
bool gemm_pipe_streamk(int64_t M, int64_t N, int64_t K, int bits);
hipError_t launch_gemm_pipe3(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                             int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st);
hipError_t launch_gemm_pipe(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st);
hipError_t launch_gemm(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                       int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st);
// 3-bit format: GEMV for M = 1 and short-row M = 2 (gemv.hip), the ring kernel up to M = 16 (skinny.hip),
// the general-shape matrix-core kernel otherwise (gemm.hip)
bool gemv3_supported(int64_t M, int64_t K);
hipError_t launch_gemv3(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                        int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm3(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                        int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st);

// Dry runs of the product dispatch.  While a KernelPlan is installed on the
// calling thread, each product launcher writes the kernel it would launch (its
// template arguments, block and grid) into it and returns hipSuccess without
// launching anything; the dispatch above it is the ordinary one.
struct KernelPlan {
  char text[160];
};
KernelPlan* active_plan();  // the calling thread's installed plan, or null
void install_plan(KernelPlan* p);
hipError_t plan_record(KernelPlan* p, const char* fmt, ...);

}  // namespace awq
