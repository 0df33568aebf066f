/*
 * libawq -- AWQ scale search, group-wise int4 weight quantizer and W4A16
 * product, for AMD Instinct MI355X (gfx950).
 *
 * What is computed follows these pages (cited by title and paragraph/section):
 *   [summary]  "AWQ: Activation-aware Weight Quantization for On-Device LLM
 *              Compression and Acceleration", fdeinterviews.com/papers/awq,
 *              paragraphs 1..10.
 *   [abstract] OpenAlex record of the GetMobile article of that title, abstract.
 *   [profile]  "AWQ: Activation-aware Weight Quantization for On-Device LLM
 *              Compression", aiexpertsdirectory.org, "Execution Profile &
 *              Computation Stack".
 *   [proof page] the same aiexpertsdirectory.org page, "Methodological &
 *              Architectural Deep-Dive".
 *
 * Notation.  A linear layer maps an input row x[K] to y[N] = W x, with W an
 * fp16 [N][K] row-major matrix (row n = output channel, like a torch Linear
 * weight).  K is the input-channel (contraction) axis.  Calibration data X is
 * fp16 [M][K] row-major.  Weights are quantized to 4-bit codes in groups of
 * `group` consecutive input channels of one output row.
 *
 * Memory.  Every pointer argument documented "device" is device memory of the
 * current HIP device; "host" pointers are ordinary host memory.  The caller
 * owns all buffers; the library allocates nothing and keeps no pointer after a
 * call returns.  Every device pointer must be 16-byte aligned: each entry
 * point checks all of its device pointers (optional ones only when given)
 * and returns AWQ_ERROR_MISALIGNED, naming the first misaligned one in
 * awq_last_error(), before anything is enqueued.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  All device work is enqueued on it in order and the calls return
 * without waiting: outputs are valid once the stream has reached that point.
 * No call synchronises the host with the device.
 *
 * Errors.  Every entry point returns an awq_status.  Argument checks happen
 * before anything is enqueued: on any status other than AWQ_OK (and
 * AWQ_ERROR_DEVICE) nothing was launched and no output was touched.
 * awq_last_error() returns a thread-local message describing the last failure
 * of the calling thread.  No call aborts or throws across this interface.
 * Non-finite values in W, X or x are outside the contract: they do not crash
 * the library, but the outputs are then unspecified.
 *
 * Thread safety.  Calls are reentrant; calls on different streams may overlap
 * when they do not share output or workspace buffers.
 */
#ifndef AWQ_H_
#define AWQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_ERROR_INVALID_VALUE = 1,         /* null pointer, bad size, bad group, bad alpha */
  AWQ_ERROR_MISALIGNED = 2,            /* a device pointer not 16-byte aligned */
  AWQ_ERROR_WORKSPACE_TOO_SMALL = 3,   /* workspace_bytes below the size query */
  AWQ_ERROR_DEVICE = 4,                /* a HIP call or kernel launch failed */
  AWQ_ERROR_NOT_IMPLEMENTED = 5
} awq_status;

/* Default quantization: 4-bit codes, group of 128 input channels.  The *_bits
 * entry points also take 3-bit codes ([summary] paragraphs 4 and 10: the
 * method is evaluated at 3 and 4 bits, 4 being the safer default). */
#define AWQ_BITS 4
#define AWQ_GROUP 128
/* Most alpha values one search accepts. */
#define AWQ_MAX_ALPHAS 64
/* Most calibration rows: keeps every per-channel sum of |x| exact in 64 bits. */
#define AWQ_MAX_CALIB_ROWS (1LL << 23)

/* ------------------------------------------------------------------------
 * Packed weight format (the "SIMD-aware weight packing" of [abstract],
 * designed here for 64-wide gfx950 waves).  For an [N][K] layer, group g:
 *
 *   packed  uint32 [N][K/8]      word w of row n holds the codes of input
 *                                channels 8w..8w+7.  Code of channel 8w+i sits
 *                                in nibble p(i) = 4*(i%2) + i/2, i.e. bits
 *                                4p..4p+3 hold, for p = 0..7, the codes of
 *                                channels 8w+{0,2,4,6,1,3,5,7}.  Masking a word
 *                                shifted right by 4j with 0x000F000F gives the
 *                                codes of channels 8w+2j and 8w+2j+1 in the two
 *                                16-bit halves.
 *   scales  fp16   [N][K/g]      step of group j of row n.
 *   zeros   uint8  [N][ceil(K/g/2)]  zero point of group j of row n in byte
 *                                j/2, low nibble for even j, high nibble for
 *                                odd j (unused high nibble = 0).
 *
 * Dequantized weight: w_hat[n][k] = (code[n][k] - zero[n][k/g]) * scale[n][k/g].
 * At g = 128 this is 4 + 2.5*8/128 = 4.156 bits per weight.
 *
 * 3-bit format (bits = 3): codes 0..7, zeros and scales as above (a zero point
 * is at most 7), and
 *   packed  uint32 [N][K/32][3]  the 32 input channels 32c..32c+31 of row n
 *                                are the words w0, w1, w2 at [n][c].  For a
 *                                channel pair p = 0..14 (channels 2p, 2p+1 of
 *                                the 32) with t = p/5, j = p%5: the code of
 *                                channel 2p sits in bits 3j..3j+2 of word t,
 *                                that of channel 2p+1 in bits 16+3j..16+3j+2.
 *                                Bit b (b = 0, 1, 2) of the codes of channels
 *                                30 and 31 sits in bits 15 and 31 of word b.
 * 3 + 2.5*8/128 = 3.156 bits per weight; K must be a multiple of 128.
 * ------------------------------------------------------------------------ */
size_t awq_packed_bytes(int64_t N, int64_t K);
/* Packed bytes at 4 or 3 bits; 0 for other widths or sizes the format cannot hold. */
size_t awq_packed_bytes_bits(int64_t N, int64_t K, int32_t bits);
size_t awq_scales_bytes(int64_t N, int64_t K, int32_t group);
size_t awq_zeros_bytes(int64_t N, int64_t K, int32_t group);

/* Workspace bytes awq_quantize needs for these sizes (pure host function). */
size_t awq_quantize_workspace_bytes(int64_t N, int64_t K, int64_t M, int32_t group, int32_t n_alpha);

/*
 * awq_channel_mean_abs -- activation statistics of the calibration set
 * ([summary] paragraphs 3 and 7: the scale of a channel comes from its
 * average activation magnitude; only activation statistics are collected).
 *
 *   X  device fp16 [M][K]   calibration rows
 *   a  device fp64 [K]      out: a[k] = (1/M) * sum_t |X[t][k]|
 *
 * The sum is exact (every fp16 |x| is a multiple of 2^-24 and the sum is kept
 * as a 64-bit count of 2^-24); only the final division rounds, so the result
 * does not depend on the order of the rows.  a doubles as the accumulator.
 * Requires 1 <= M <= AWQ_MAX_CALIB_ROWS, K >= 8, K % 8 == 0.
 */
int awq_channel_mean_abs(const void* X, int64_t M, int64_t K, double* a, void* stream);

/*
 * awq_pack -- quantize W * diag(s) group-wise to int4 and write the packed
 * format above.  With s == NULL the weights are quantized unscaled (plain
 * round-to-nearest, the baseline of [summary] paragraph 4).
 *
 *   W       device fp16 [N][K]
 *   s       device fp32 [K] or NULL   per-input-channel factor
 *   packed, scales, zeros   device outputs, sizes from the queries above
 *
 * Per group (float32 arithmetic, round-to-nearest-even everywhere):
 *   v = w * s;  lo = min(0, min v);  hi = max(0, max v)
 *   step = max((hi - lo) / 15, 2^-14);  scale = fp16(step)
 *   zero = clamp(rint(-lo / scale), 0, 15);  code = clamp(rint(v / scale) + zero, 0, 15)
 * Requires N >= 1, K % group == 0, group == AWQ_GROUP.
 */
int awq_pack(const void* W, const float* s, int64_t N, int64_t K, int32_t group,
             void* packed, void* scales, void* zeros, void* stream);
/* awq_pack at `bits` = 4 (as above) or 3 (15 in the formulas above becomes 7,
 * and the 3-bit format is written).  Requires bits == 4 or 3. */
int awq_pack_bits(const void* W, const float* s, int64_t N, int64_t K, int32_t group, int32_t bits,
                  void* packed, void* scales, void* zeros, void* stream);

/*
 * awq_quantize -- the activation-aware scale search of [summary] paragraph 3
 * (also [abstract]) for one linear layer, then quantize-and-pack at the best
 * alpha.
 *
 *   W          device fp16 [N][K]      layer weight
 *   X          device fp16 [M][K]      calibration rows entering the layer
 *   alphas     host fp32 [n_alpha]     grid, each finite and >= 0
 *   packed, scales, zeros              device outputs (format above) at alpha*
 *   s          device fp32 [K]         out: s at alpha*
 *   best_alpha device int32 [1]        out: index of alpha* in `alphas`
 *   loss       device fp64 [n_alpha] or NULL   out: L(alpha_i)
 *   workspace  device, workspace_bytes >= awq_quantize_workspace_bytes(...)
 *
 * For each alpha_i: a = awq_channel_mean_abs(X); s_k = fp32(a_k ^ alpha_i)
 * evaluated in fp64 (s_k = 1 where a_k = 0); quantize W diag(s) as awq_pack;
 * E = w_hat / s - w; L_i = ||X E^T||_F^2 / (M N), the mean squared change of
 * the layer's output on the calibration rows.  For M < K it is evaluated
 * directly (Y = X E^T with E in fp32 on the fp32 matrix cores); for M >= K
 * through G = X^T X as sum_n E_n G E_n^T (G accumulated in fp64, then both
 * factors rescaled per channel by powers of two and split into fp16 hi + lo
 * pairs for the fp16 matrix cores).  Partial sums are reduced in fp64 in a
 * fixed order; L agrees with an fp64 evaluation to about 1e-7 relative.  The
 * Gram form assumes |E_nk| * sqrt(G_kk) < 2^15 (far above any 4-bit
 * quantization error of realistic weights).  alpha* is the first index with
 * the smallest L.  The caller then feeds x / s (rounded to fp16) to awq_gemm.
 * Requires 1 <= n_alpha <= AWQ_MAX_ALPHAS, 1 <= M <= AWQ_MAX_CALIB_ROWS,
 * group == AWQ_GROUP, K % group == 0.
 */
int awq_quantize(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group,
                 const float* alphas, int32_t n_alpha,
                 void* packed, void* scales, void* zeros, float* s,
                 int32_t* best_alpha, double* loss,
                 void* workspace, size_t workspace_bytes, void* stream);
/* awq_quantize at `bits` = 4 (as above) or 3 (the quantizer and format of
 * awq_pack_bits); the workspace does not depend on bits. */
int awq_quantize_bits(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group,
                      int32_t bits, const float* alphas, int32_t n_alpha,
                      void* packed, void* scales, void* zeros, float* s,
                      int32_t* best_alpha, double* loss,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * awq_quantize_shared -- awq_quantize_bits for layers that read the same input
 * (q/k/v, gate/up): with reuse_statistics = 1 the statistics of X (the channel
 * means a and, for M >= K, the scaled fp16 split of G = X^T X) are taken from
 * `workspace`, where the previous awq_quantize* call on this workspace left
 * them, instead of being recomputed; everything after them (s(alpha), the
 * errors, the losses, the pack) runs as in awq_quantize_bits, so the outputs
 * are identical.  The caller guarantees that the previous call on this
 * workspace had the same X contents, M and K (N, bits, the alpha grid and W
 * may differ) and that the workspace was not written in between; otherwise the
 * outputs are unspecified.  reuse_statistics = 0 is awq_quantize_bits.  The
 * workspace must cover awq_quantize_workspace_bytes of this call.
 */
int awq_quantize_shared(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group, int32_t bits,
                        const float* alphas, int32_t n_alpha, int32_t reuse_statistics,
                        void* packed, void* scales, void* zeros, float* s,
                        int32_t* best_alpha, double* loss,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * awq_gemm -- the W4A16 product that 4-bit decoding runs on ([summary]
 * paragraphs 1 and 6: decoding is memory-bound, 4-bit weights cut its
 * traffic about 4x; [profile]: W4A16 GEMM kernels).  The int4 weights are
 * dequantized on the fly in registers ([abstract]).
 *
 *   x       device fp16 [M][K]  activations (already divided by s)
 *   packed, scales, zeros       device, format above
 *   y       device fp16 [M][N]  out: y[m][n] = sum_k x[m][k] * w_hat[n][k]
 *
 * Accumulation is fp32 and y is rounded to fp16 once.  M = 1, and M = 2 with
 * K < 16384: vector-ALU GEMV on (code - zero), exact in fp16, every product
 * with x exact in fp32, the group scale applied to each 32-code partial sum in
 * fp32 (so a row whose codes all equal their zero points gives y = 0 exactly).
 * Other M <= 16, and
 * 17 <= M <= 64 on the layer shapes the matrix-core decode kernels serve
 * (N <= 8192; N <= 12288 with K > 4096, K >= 8192 above M = 32; K <= 4096 or
 * K >= 8192 up to M = 32): matrix-core kernels on (code - zero), exact in fp16, with fp32 sums per
 * 128-channel group and the group scale applied in fp32, so no dequantized
 * weight is rounded.  Other
 * M >= 17: the pipelined matrix-core GEMM multiplies the dequantized weight
 * (code - zero) * scale rounded once to fp16 (relative error <= 2^-11 per
 * weight; a weight with |code - zero| * scale above 65504 overflows to inf),
 * or, where the block's scales do not fit its LDS (K above about 32K), the
 * general-shape kernel with the exact arithmetic above.
 * Requires M >= 1, 1 <= N < 2^31, K % group == 0, K <= 2^20, group == AWQ_GROUP.
 */
int awq_gemm(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
             int64_t M, int64_t N, int64_t K, int32_t group, void* stream);
/* awq_gemm on the format written at `bits` = 4 (awq_gemm itself) or 3.  At 3
 * bits: M = 1, and M = 2 with K < 16384, run the vector-ALU GEMV with the
 * arithmetic stated above (exact code - zero, every product exact in
 * fp32); other M <= 64 the matrix-core decode kernel on exact
 * (code - zero) with the group scale applied in fp32; M > 64, and M > 32 on
 * layers wider than 12288 rows or with K <= 4096 (N > 8192), the pipelined
 * matrix-core GEMM with the 4-bit arithmetic above (the dequantized weight
 * rounded once to fp16), or, where the block's scales do not fit its LDS, the
 * general-shape kernel on exact (code - zero).  Requires bits == 4 or 3 and
 * M <= 65535 * 64 at 3 bits. */
int awq_gemm_bits(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                  int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, void* stream);
/* awq_gemm_ws -- awq_gemm_bits with a workspace, in which the matrix-core GEMM
 * can split its work evenly over the compute units instead of giving each block
 * whole output tiles (stream-K: block v of P takes the v-th P-th of the
 * (tile, 128-channel group) pairs; a tile whose groups are split between blocks
 * is summed by the block that finishes it last, which adds the blocks' fp32
 * partials in the order of their K ranges, so y is deterministic).  The split
 * applies for M > 32 when whole tiles would leave at least half of the compute
 * units idle in their last round and every unit gets at least 8 groups; the
 * workspace size query says whether it does (0 bytes: it does not, and the call
 * is awq_gemm_bits).  The split changes the scheduling, not the product: it is
 * awq_gemm's ([summary] paragraph 9, the batched regime).
 *   workspace        device, >= awq_gemm_workspace_bytes(M, N, K, bits) bytes
 *                    (may be NULL when that is 0); it holds the blocks' partial
 *                    tiles and, after them, tile counters that must be zero
 *                    before the first call on a new workspace: clear it once
 *                    after allocating it (every call leaves the counters zero,
 *                    so the workspace then serves calls of any size)
 *   other arguments  as awq_gemm_bits
 * Calls that share a workspace must not overlap in time (one stream, or ordered
 * by events).  Where the split applies, y agrees with awq_gemm_bits to fp32
 * rounding (the sum over K is grouped differently), and a layer stored with
 * others' rows concatenated (fused q/k/v) may differ from the separate layers in
 * the last bit; elsewhere y is awq_gemm_bits's bit for bit.
 * Errors: those of awq_gemm_bits; AWQ_ERROR_INVALID_VALUE for a NULL workspace
 * that is needed, AWQ_ERROR_WORKSPACE_TOO_SMALL, AWQ_ERROR_MISALIGNED for a
 * workspace not 16-byte aligned. */
size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits);
int awq_gemm_ws(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, void* workspace,
                size_t workspace_bytes, void* stream);
/* awq_gemm_ws_kernel -- awq_gemm_kernel for awq_gemm_ws (given a large enough
 * workspace); the text ends in " stream-K" where the split applies. */
int awq_gemm_ws_kernel(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, char* out, size_t out_bytes);

/* awq_gemm_kernel -- the kernel awq_gemm_bits launches for an M x K input and
 * N x K weights at `bits`: a dry run of the same dispatch that launches
 * nothing and touches no device (host-only; it works without a GPU).  Writes
 * the kernel's name with its template arguments, block and grid, for example
 * "ring_kernel<4,1,1,2,32> block=256 grid=257", NUL-terminated and truncated
 * to `out_bytes` (160 bytes always suffice), to `out` (host).  For tests that
 * must reach every branch of the dispatch, and for diagnostics.  Returns
 * AWQ_OK, or AWQ_ERROR_INVALID_VALUE for sizes awq_gemm_bits refuses (then
 * `out` holds the empty string) or a NULL `out`.
 */
int awq_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, char* out, size_t out_bytes);

/*
 * The input side of the per-channel scaling ([summary] paragraph 3: a weight
 * channel scaled up by s has its input divided by s, so the product keeps its
 * value).  awq_gemm takes x already divided; these calls do the division on
 * the device.  The scaled input is fp16(x / s): one IEEE fp32 division of
 * fp32(x) by s (correctly rounded), rounded once more to fp16 (round to
 * nearest even).
 *
 * awq_scale_input -- xs[m][k] = fp16(fp32(x[m][k]) / s[k]).
 *   x      device fp16 [M][K]
 *   s      device fp32 [K]   per-channel scale (awq_quantize's s)
 *   xs     device fp16 [M][K]   out (may not overlap x)
 * Requires 1 <= M <= 2^22, K % 8 == 0, 8 <= K <= 2^20.
 */
int awq_scale_input(const void* x, const float* s, int64_t M, int64_t K, void* xs, void* stream);

/*
 * awq_gemm_scaled -- y = awq_scale_input(x, s) times w_hat^T: the scaled input
 * is written to `workspace` (device, awq_gemm_scaled_workspace_bytes =
 * M * K * 2 bytes rounded up to 256), then the product of awq_gemm_bits runs
 * on it, so y equals awq_gemm_bits on awq_scale_input's output bit for bit.
 * (Dividing inside the decode GEMV's own x load instead repeats the division
 * in every block, since each block spans all of K; done exactly that measured
 * slower than the separate launch on every decode layer shape.)
 *   x      device fp16 [M][K]   activations, not divided by s
 *   s      device fp32 [K]      per-channel scale
 *   other arguments as awq_gemm_bits
 * Requires what awq_gemm_bits requires.
 */
size_t awq_gemm_scaled_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits);
int awq_gemm_scaled(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                    void* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * awq_gemm_scaled_static -- awq_gemm_scaled with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The call allocates
 * nothing: the scaled input goes to a static device array of
 * AWQ_STATIC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call made with that device current).  y equals awq_gemm_scaled's
 * bit for bit.  Every call on one device shares that device's array, which
 * keeps the last call's contents (each call writes the part it then reads, so
 * nothing needs clearing): calls that overlap on one device -- on different
 * streams, or from threads with no ordering between them -- race and give
 * unspecified results; calls ordered on one stream do not.
 * Requires awq_gemm_scaled_workspace_bytes(M, N, K, bits) <=
 * AWQ_STATIC_SCRATCH_BYTES (M * K <= 2^23 halfs; otherwise
 * AWQ_ERROR_INVALID_VALUE) and what awq_gemm_scaled requires.
 */
#define AWQ_STATIC_SCRATCH_BYTES (16u << 20)
int awq_gemm_scaled_static(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                           void* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, void* stream);

/*
 * awq_unpack -- logical view of the packed format, for checking it.
 *   codes     device uint8 [N][K]     out: code of every weight
 *   zeros_u8  device uint8 [N][K/g]   out: zero point of every group
 */
int awq_unpack(const void* packed, const void* zeros, int64_t N, int64_t K, int32_t group,
               uint8_t* codes, uint8_t* zeros_u8, void* stream);
/* awq_unpack of the format written at `bits` = 4 or 3. */
int awq_unpack_bits(const void* packed, const void* zeros, int64_t N, int64_t K, int32_t group, int32_t bits,
                    uint8_t* codes, uint8_t* zeros_u8, void* stream);

/*
 * awq_keep_fp16_ablation -- the observation AWQ starts from ([summary]
 * paragraph 2; [proof page], methodological paragraph): keeping a few input
 * channels of a layer in 16-bit while rounding the rest recovers most of the
 * rounding loss, but only when the channels are chosen by activation
 * magnitude; chosen by weight magnitude they do about as well as at random.
 *
 *   W, X        device fp16 [N][K] weight and [M][K] calibration rows
 *   bits        4 or 3
 *   n_keep      channels kept, 0 <= n_keep <= K
 *   random_keep device int32 [n_keep]   the caller's random choice of channels
 *                                       (entries outside [0, K) are ignored)
 *   keep_act    device int32 [n_keep]   out: channels of largest mean |x| over
 *                                       X's rows, largest first
 *   keep_wt     device int32 [n_keep]   out: channels of largest mean |w| over
 *                                       W's rows, largest first
 *   loss        device fp64 [4]         out: output MSE on X with no channel
 *                                       kept, keep_act, keep_wt, random_keep
 *   workspace   device, >= awq_ablation_workspace_bytes(N, K, M, group)
 *
 * W is quantized group-wise exactly as awq_pack with s = NULL (plain
 * round-to-nearest); the kept channels' weights are then used unrounded (they
 * stay in their groups' ranges, so every choice shares the same steps).  The
 * loss is that of awq_quantize, L = ||X E^T||_F^2 / (M N) with E = w_hat - w
 * and E = 0 on the kept channels, in the same direct or Gram form.  Equal
 * magnitudes are ordered by the lower channel index; the magnitudes are exact
 * sums (as awq_channel_mean_abs), so the choice is reproducible.
 * Requires 1 <= M, N <= AWQ_MAX_CALIB_ROWS, group == AWQ_GROUP, K % group == 0.
 */
size_t awq_ablation_workspace_bytes(int64_t N, int64_t K, int64_t M, int32_t group);
int awq_keep_fp16_ablation(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group,
                           int32_t bits, int32_t n_keep, const int32_t* random_keep,
                           int32_t* keep_act, int32_t* keep_wt, double* loss,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Message for a status code; message for the calling thread's last failure. */
const char* awq_status_string(int status);
const char* awq_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int awq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_H_ */
