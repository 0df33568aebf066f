/*
 * libawq_ceilings -- measurement kernels for gfx950 that bound what the
 * libawq kernels can reach on one device: a streaming read (the HBM ceiling
 * the decode GEMV is measured against), the same read ending each block with
 * one dependent store (the decode GEMV's shape), and a dense fp16 matrix-core
 * loop (the MFMA ceiling of the GEMM and the search contractions).  They
 * compute nothing of the method; only bench.py's ceiling leg calls them.
 *
 * Memory and streams follow libawq (include/awq.h): device pointers of the
 * current device, 16-byte aligned, owned by the caller; work enqueued on
 * `stream` (a hipStream_t as void*), no host synchronisation.  Each call
 * returns 0 on success, 1 for invalid arguments (nothing launched), 4 when the
 * launch fails.
 */
#ifndef AWQ_CEILINGS_H_
#define AWQ_CEILINGS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * awq_ceiling_stream_read -- reads `bytes` bytes of `src` once with 16-byte
 * non-temporal loads (the decode GEMV's weight loads).  Each thread issues its
 * `loads_per_thread` loads (1, 2 or 4; the 256 threads of a block cover
 * consecutive pieces) before using any, and the grid spans the whole range: one
 * round trip per thread, as the decode GEMV makes.  What a thread read is
 * folded into one word, stored to sink[block % 1024] only when it equals a
 * fixed pattern (practically never), so no load is dead code.
 *   src    device, bytes % 16 == 0, bytes >= 16
 *   sink   device uint32 [1024]
 */
int awq_ceiling_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t loads_per_thread, void* stream);

/*
 * awq_ceiling_stream_read_store -- the read of awq_ceiling_stream_read, with
 * each 256-thread block finishing as a decode GEMV block does: its threads'
 * folded words are combined across the block (shuffles, then LDS after a
 * barrier) and one 4-byte store per block writes the result to out[block].
 * The difference from awq_ceiling_stream_read is what a kernel that writes its
 * outputs after all of its loads pays for that dependent store.
 *   out        device uint32 [out_words], out_words >= the number of blocks,
 *              ceil(bytes / (4096 loads_per_thread))
 */
int awq_ceiling_stream_read_store(const void* src, size_t bytes, uint32_t* out, size_t out_words,
                                  int32_t loads_per_thread, void* stream);

/*
 * awq_ceiling_mfma_f16 -- each of `blocks` blocks of 4 * waves_per_simd waves
 * (256 or 512 threads: one or two waves per SIMD when one block runs per
 * compute unit) runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_f16
 * on register operands and stores one float per wave to sink.
 * Work: blocks * 4 * waves_per_simd * iters * 8 * 32768 flops.
 *   sink   device fp32 [blocks * 4 * waves_per_simd]
 * Requires 1 <= blocks <= 65536, 1 <= iters <= 2^20, waves_per_simd 1 or 2.
 */
int awq_ceiling_mfma_f16(float* sink, int32_t blocks, int32_t iters, int32_t waves_per_simd, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_CEILINGS_H_ */
