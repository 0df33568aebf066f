// Output-MSE of one alpha: L = ||X E^T||_F^2 / (M N) = sum_n E_n G E_n^T / (M N)
// with G = X^T X, E = w_hat / s - w.  The search picks the alpha whose
// quantized layer changes the layer's output least on the calibration rows
// ("AWQ: Activation-aware Weight Quantization for On-Device LLM Compression and
// Acceleration", fdeinterviews.com/papers/awq, paragraph 3: grid search over
// alpha on a small calibration set, no backpropagation).
//
// Precision plan (exact rescaling, then a 22-bit split for the fp16 matrix
// cores).  With a power of two 2^e_k per channel (e_k ~ log2 sqrt(G_kk)),
//   G'_kj = G_kj 2^(-e_k - e_j),  E'_nk = E_nk 2^(e_k),  sum_n E'_n G' E'_n^T = sum_n E_n G E_n^T
// exactly, and |G'| <= ~2 (Cauchy-Schwarz) while E' stays well inside fp16
// range.  Each of E', G' is stored as an fp16 pair hi + lo (hi = fp16(v),
// lo = fp16(v - hi)), and products are formed on v_mfma_f32_32x32x16_f16 as
// hi.hi + hi.lo + lo.hi with fp32 accumulation (the dropped lo.lo term is
// ~2^-22 relative).  Block partial sums go to fp64 and are reduced in a fixed
// order, so the result is deterministic; it agrees with an fp64 evaluation to
// about 1e-7 relative.
//
// Symmetry.  With the channels cut into 256-wide blocks I, J, and G symmetric,
//   sum_n E_n G E_n^T = sum_n sum_{I <= J} E_{n,I} G''_{I,J} E_{n,J}^T
// where G'' = 2 G' on the blocks off the diagonal and G' on it (the doubling is
// exact): only the block-upper triangle is contracted, about half of the full
// product's work.  The split kernel stores G'' directly.
//
// This Gram form is used when M >= K; for M < K see the direct form below.
//
// Work split: for an n-tile (256 rows of E') and a channel block J, the segment
// T = E' G''[., J] contracts channels 0 .. 256 (J + 1) - 1 in stages of 32.  All
// segments, n-tile by n-tile and within one the longest J first, form one line
// of stages, and each of kLossBlocks persistent blocks (one per compute unit)
// takes an equal run of it; a run that crosses segment boundaries contracts
// each piece into a 256 x 256 tile of T and adds sum E'[n][j] T[n][j] over the
// tile to the block's partial.  The loss is linear in T, so the pieces of one
// segment simply add: every compute unit does the same number of stages and
// no fix-up pass is needed.  Block b's run index puts the runs of one XCD
// (b % 8) side by side (mostly whole n-tiles, which then share E' through that
// XCD's L2).
#include "awq_common.h"
#include "awq_internal.h"
#include "mfma_pipe.h"

namespace awq {

constexpr int kFT = 256;     // tile of T: 256 rows n x 256 columns j
// Stage width, measured on the 7B shapes: two 32-channel stages beat four
// 16-channel stages by 5-9 % (half the barriers).
constexpr int kFKS = 32;                     // channels per pipeline stage
constexpr int kFStages = 2;                  // two stages of 32 channels: 128 KB of LDS
constexpr int kFLoads = 4 * (kFT / (512 / kFKS) / 8);  // direct loads per wave per stage

constexpr int kLossBlocks = 256;  // persistent blocks: one per compute unit (128 KB of LDS each)

static int64_t full_tiles_n(int64_t N) { return (N + kFT - 1) / kFT; }
static int64_t full_tiles_j(int64_t K) { return (K + kFT - 1) / kFT; }

// Stages of channel block J's segment: channels 0 .. min(256 (J + 1), K) - 1.
__host__ __device__ inline int seg_stages(int J, int64_t K) {
  const int64_t c = (int64_t)(J + 1) * kFT < K ? (int64_t)(J + 1) * kFT : K;
  return (int)(c / kFKS);
}

// Stages of one n-tile's segments.
__host__ __device__ inline int64_t stages_per_ntile(int64_t K) {
  int64_t u = 0;
  for (int J = 0; J < (int)full_tiles_j(K); ++J) u += seg_stages(J, K);
  return u;
}

int64_t loss_partial_count(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return kLossBlocks;
}

// e_k = floor(log2(G_kk) / 2), 0 where G_kk is 0 (a channel that is zero in every row).
__global__ void channel_exponent_kernel(const float* __restrict__ G, int64_t K, int32_t* __restrict__ e) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const float d = G[k * K + k];
  e[k] = (d > 0.0f) ? (ilogbf(d) >> 1) : 0;
}

// Ghi/Glo = split of G''_kj = G_kj 2^(-e_k - e_j), doubled when k and j lie in
// different 256-channel blocks (see the symmetry note above); the scaling is
// exact in fp32.
__global__ void gram_split_kernel(const float* __restrict__ G, const int32_t* __restrict__ e, int64_t K,
                                  f16* __restrict__ Ghi, f16* __restrict__ Glo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= K * K) return;
  const int64_t k = i / K, j = i - k * K;
  const int off_diag = (k / kFT) != (j / kFT) ? 1 : 0;
  const float v = ldexpf(G[i], off_diag - (e[k] + e[j]));
  const f16 hi = (f16)v;
  Ghi[i] = hi;
  Glo[i] = (f16)(v - (float)hi);
}

hipError_t launch_gram_split(const float* G, int64_t K, int32_t* e, void* Ghi, void* Glo, hipStream_t st) {
  channel_exponent_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(G, K, e);
  const int64_t n = K * K;
  gram_split_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(G, e, K, reinterpret_cast<f16*>(Ghi),
                                                                              reinterpret_cast<f16*>(Glo));
  return hipGetLastError();
}

// Block: 512 threads = 8 waves (two per SIMD) in 2 (j) x 4 (n), wave tile
// 128 j x 64 n.  The matrix cores form D[j][n] = sum_k G'[j][k] E'[n][k] =
// T[n][j] (G' is symmetric): A operand = rows j of G', B operand = rows n of
// E', three MFMAs (hi.hi, hi.lo, lo.hi) per fragment pair.  D register r of
// lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32], so a lane's registers 4q..4q+3
// are 4 consecutive j of one n and the epilogue reads E'[n][j..j+3] with one
// 8-byte load per fp16 half.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void loss_full_kernel(const f16* __restrict__ Ehi, const f16* __restrict__ Elo, const f16* __restrict__ Ghi,
                      const f16* __restrict__ Glo, int64_t N, int64_t K, int nt, int jt, int64_t per_n,
                      double* __restrict__ partial) {
  constexpr int D = kFStages - 1;  // stages in flight ahead of the one computed
  // The only LDS variable of the kernel: with a second one the compiler tags every LDS
  // access with alias scopes, and then waits for all outstanding direct loads before
  // each fragment read (it cannot tell the stage being filled from the one being read),
  // which would serialize the pipeline.  The final reduction reuses the stage buffers.
  __shared__ __attribute__((aligned(16))) f16 lds[kFStages][4][kFT * kFKS];  // 131,072 B
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wj = wave >> 2, wn = wave & 3, l32 = lane & 31;

  // this block's run [pos, end) of the line of stages (gridDim.x is a multiple of 8)
  const int64_t total = (int64_t)nt * per_n;
  const int64_t r = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  int64_t pos = total * r / gridDim.x;
  const int64_t end = total * (r + 1) / gridDim.x;
  // the segment holding pos: n-tile nb, channel block J (longest first), stage s0 in it
  int nb = (int)(pos / per_n), J = jt - 1;
  int64_t s0 = pos - (int64_t)nb * per_n;
  while (s0 >= seg_stages(J, K)) s0 -= seg_stages(J--, K);

  double sum = 0.0;  // this lane's share of the block's partial
  while (pos < end) {
    const int64_t seg = seg_stages(J, K);
    const int64_t S0 = s0, S = (seg - s0) < (end - pos) ? seg : s0 + (end - pos);  // stages [S0, S) of segment
    const int64_t j0 = (int64_t)J * kFT, n0 = (int64_t)nb * kFT;

    TilePlan<kFT, 8, kFKS> pgh, pgl, peh, pel;
    pgh.init(Ghi, K, j0, K, wave, lane);
    pgl.init(Glo, K, j0, K, wave, lane);
    peh.init(Ehi, K, n0, N, wave, lane);
    pel.init(Elo, K, n0, N, wave, lane);
    // past the last stage the tail re-reads stage S - 1 into the free slot; stage s
    // goes to ring slot (s - S0) % kFStages
    auto issue = [&](int64_t st) {
      const int64_t k0 = (st < S ? st : S - 1) * kFKS;
      const int slot = (int)((st - S0) % kFStages);
      pgh.issue(lds[slot][0], k0);
      pgl.issue(lds[slot][1], k0);
      peh.issue(lds[slot][2], k0);
      pel.issue(lds[slot][3], k0);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

    lds_barrier();  // every wave is done with the ring before it is refilled
    for (int t = 0; t < D; ++t) issue(S0 + t);
    for (int64_t st = S0; st < S; ++st) {
      wait_vmcnt<(D - 1) * kFLoads>();  // stage st has landed; stages st+1 .. st+D-1 may be pending
      lds_barrier();                     // ... for every wave; stage st - 1 is no longer read
      issue(st + D);
      const int slot = (int)((st - S0) % kFStages);
      const f16* Gh = lds[slot][0];
      const f16* Gl = lds[slot][1];
      const f16* Eh = lds[slot][2];
      const f16* El = lds[slot][3];
      // The stage's E' fragments are read up front; the G'' fragments of step i + 1
      // (channel half hk, 32-row block a) are read while the matrix cores run step i.
      constexpr int HK = kFKS / 16, STEPS = HK * 4;
      f16x8 eh[HK][2], el[HK][2], gh[2], gl[2];
#pragma unroll
      for (int hk = 0; hk < HK; ++hk)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          eh[hk][b] = frag32(Eh, wn * 64 + b * 32 + l32, 2 * hk + (lane >> 5));
          el[hk][b] = frag32(El, wn * 64 + b * 32 + l32, 2 * hk + (lane >> 5));
        }
      auto load_g = [&](int i, int buf) {
        const int c = 2 * (i >> 2) + (lane >> 5), row = wj * 128 + (i & 3) * 32 + l32;
        gh[buf] = frag32(Gh, row, c);
        gl[buf] = frag32(Gl, row, c);
      };
      load_g(0, 0);
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        if (i + 1 < STEPS) load_g(i + 1, (i + 1) & 1);
        const int hk = i >> 2, a = i & 3, cb = i & 1;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gh[cb], eh[hk][b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gh[cb], el[hk][b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(gl[cb], eh[hk][b], acc[a][b], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep each step's reads and MFMAs within the step
      }
    }
    wait_vmcnt<0>();  // the tail's redundant loads land before the ring is reused or the block exits

    // sum over the tile of E'[n][j] * T[n][j], E' = hi + lo in fp32.  For each of its two
    // rows n the lane loads its 16 E' pairs before using any (two round trips to memory;
    // all 32 at once would not fit beside the accumulators, and the compiler then waited
    // for the loads one by one); rows past N and channels past K (all 4 of a quad or none,
    // K % 128 == 0) read a valid element and are dropped from the sum.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      int64_t nl = n0 + wn * 64 + b * 32 + l32;
      const bool nlive = nl < N;
      nl = nlive ? nl : N - 1;
      u32x2 hv[4][4], lv[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int64_t j = j0 + wj * 128 + a * 32 + 8 * q + 4 * (lane >> 5);
          j = j < K ? j : K - 4;
          hv[a][q] = *reinterpret_cast<const u32x2*>(Ehi + nl * K + j);
          lv[a][q] = *reinterpret_cast<const u32x2*>(Elo + nl * K + j);
        }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t j = j0 + wj * 128 + a * 32 + 8 * q + 4 * (lane >> 5);
          if (!nlive || j >= K) continue;
          const f16x2 h01 = as_f16x2(hv[a][q].x), h23 = as_f16x2(hv[a][q].y);
          const f16x2 l01 = as_f16x2(lv[a][q].x), l23 = as_f16x2(lv[a][q].y);
          const float e[4] = {(float)h01.x + (float)l01.x, (float)h01.y + (float)l01.y,
                              (float)h23.x + (float)l23.x, (float)h23.y + (float)l23.y};
#pragma unroll
          for (int u = 0; u < 4; ++u) sum += (double)e[u] * (double)acc[a][b][4 * q + u];
        }
    }

    // next segment: the next channel block of this n-tile, or the next n-tile
    pos += S - S0;
    s0 = 0;
    if (--J < 0) {
      J = jt - 1;
      ++nb;
    }
  }

  sum = wave_sum(sum);
  double* red = reinterpret_cast<double*>(&lds[0][0][0]);
  __syncthreads();  // every wave is past its last fragment read
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    double v = 0.0;
    for (int w = 0; w < 8; ++w) v += red[w];
    partial[blockIdx.x] = v;
  }
}

hipError_t launch_loss_partials(const void* Ehi, const void* Elo, const void* Ghi, const void* Glo, int64_t N,
                                int64_t K, double* partial, hipStream_t st) {
  const int nt = (int)full_tiles_n(N), jt = (int)full_tiles_j(K);
  loss_full_kernel<<<dim3((unsigned)kLossBlocks), dim3(512), 0, st>>>(
      reinterpret_cast<const f16*>(Ehi), reinterpret_cast<const f16*>(Elo), reinterpret_cast<const f16*>(Ghi),
      reinterpret_cast<const f16*>(Glo), N, K, nt, jt, stages_per_ntile(K), partial);
  return hipGetLastError();
}

// Direct form for M < K (few calibration rows, where X^T X is far from full
// rank and its split would lose accuracy): L = sum_{t,n} Y_tn^2 / (M N) with
// Y = X E^T, E in fp32 and X (fp16, exact in fp32) on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  Block: 64 rows t x 64 rows n, 4 waves in 2 x 2,
// each 32 x 32 as 2 x 2 MFMA tiles; 16x16x4 fp32 layouts: A lane l holds
// A[l%16][l/16], B lane l holds B[l/16][l%16], D register r of lane l is
// D[4*(l/16)+r][l%16].
constexpr int kDT = 64, kDKS = 16;

int64_t loss_direct_partial_count(int64_t M, int64_t N) { return ((M + kDT - 1) / kDT) * ((N + kDT - 1) / kDT); }

__global__ __launch_bounds__(256) void loss_direct_kernel(const f16* __restrict__ X, const float* __restrict__ E,
                                                          int64_t M, int64_t N, int64_t K,
                                                          double* __restrict__ partial) {
  __shared__ float As[kDT][kDKS + 1];
  __shared__ float Bs[kDT][kDKS + 1];
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * kDT, n0 = (int64_t)blockIdx.x * kDT;
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  const bool alive = t0 + lr < M, blive = n0 + lr < N;
  const f16* Ap = X + (alive ? t0 + lr : M - 1) * K + lc;
  const float* Bp = E + (blive ? n0 + lr : N - 1) * K + lc;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < K; k0 += kDKS) {
    const uint2 araw = *reinterpret_cast<const uint2*>(Ap + k0);
    const float4 bv = *reinterpret_cast<const float4*>(Bp + k0);
    const f16x2 a01 = as_f16x2(araw.x), a23 = as_f16x2(araw.y);
    __syncthreads();
    As[lr][lc + 0] = alive ? (float)a01.x : 0.f;
    As[lr][lc + 1] = alive ? (float)a01.y : 0.f;
    As[lr][lc + 2] = alive ? (float)a23.x : 0.f;
    As[lr][lc + 3] = alive ? (float)a23.y : 0.f;
    Bs[lr][lc + 0] = blive ? bv.x : 0.f;
    Bs[lr][lc + 1] = blive ? bv.y : 0.f;
    Bs[lr][lc + 2] = blive ? bv.z : 0.f;
    Bs[lr][lc + 3] = blive ? bv.w : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kDKS; kk += 4) {
      float a_[2], b_[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) a_[a] = As[wi * 32 + a * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int b = 0; b < 2; ++b) b_[b] = Bs[wj * 32 + b * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_[a], b_[b], acc[a][b], 0, 0, 0);
    }
  }
  double sum = 0.0;  // rows t >= M and n >= N hold zeros
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += (double)acc[a][b][r] * (double)acc[a][b][r];
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_loss_direct(const void* X, const float* E, int64_t M, int64_t N, int64_t K, double* partial,
                              hipStream_t st) {
  dim3 grid((unsigned)((N + kDT - 1) / kDT), (unsigned)((M + kDT - 1) / kDT));
  loss_direct_kernel<<<grid, dim3(256), 0, st>>>(reinterpret_cast<const f16*>(X), E, M, N, K, partial);
  return hipGetLastError();
}

// loss[0] = (sum of partial[0..count)) / mn, summed in a fixed order.
__global__ __launch_bounds__(256) void loss_reduce_kernel(const double* __restrict__ partial, int64_t count,
                                                          double mn, double* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += 256) s += partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = red[0] / mn;
}

hipError_t launch_loss_reduce(const double* partial, int64_t count, double mn, double* loss, hipStream_t st) {
  loss_reduce_kernel<<<dim3(1), dim3(256), 0, st>>>(partial, count, mn, loss);
  return hipGetLastError();
}

// First index of the smallest loss.
__global__ void argmin_kernel(const double* __restrict__ loss, int n, int32_t* __restrict__ best) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int b = 0;
  for (int i = 1; i < n; ++i)
    if (loss[i] < loss[b]) b = i;
  best[0] = b;
}

hipError_t launch_argmin(const double* loss, int n, int32_t* best, hipStream_t st) {
  argmin_kernel<<<dim3(1), dim3(64), 0, st>>>(loss, n, best);
  return hipGetLastError();
}

}  // namespace awq
