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
// Two kernels share that arithmetic.  In both, a block owns 16*RW weight rows
// and all of K, its W waves split the K groups, and the waves' partial tiles
// are summed through LDS in a fixed order, so results are deterministic.
//
// The register-staged kernel (skinny_kernel): wave w takes groups w, w+W, ....
// For one group a wave loads 16 B per lane: lane l reads the (l/16)-th 16-byte
// quarter of the group's 64 B in row l%16, so one load instruction fetches 16
// rows x 64 B.  All loads of a batch of P groups (and their x fragments, when
// they fit in registers) are issued before any is used.  It serves the shapes
// the ring kernel declines because the block's scales and zeros leave its
// rings no LDS (K beyond ~130,000 at 17 <= M <= 64, ~260,000 at M <= 16), and
// M = 1 beyond the GEMV's K = 32768.
//
// The ring kernel (ring_kernel, 3 <= M <= 16, and M = 2 on rows of 16384
// channels or more) moves weights and x fragments
// from memory straight into per-wave LDS rings; it is described with its code.
#include "awq_common.h"
#include "awq_internal.h"
#include "mfma_pipe.h"

namespace awq {

constexpr int kSkinnyMaxWaves = 8;

// Waves per block: about P groups per wave, at most kSkinnyMaxWaves.  It is a
// function of K alone, so the kernel derives it from its arguments (which the
// hardware preloads into registers) instead of reading the dispatch packet.
template <int P>
__host__ __device__ inline int skinny_waves(int64_t K) {
  const int64_t w = (K / kGroup + P - 1) / P;
  return w < 1 ? 1 : (w > kSkinnyMaxWaves ? kSkinnyMaxWaves : (int)w);
}

template <int RW, int P, int MT>
__global__ __launch_bounds__(512) void skinny_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                     const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                     f16* __restrict__ y, int M, int N32, int K32) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int64_t N = N32, K = K32;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  // The batch's x fragments are loaded together with its weights, before the
  // first wait, when they fit in registers; otherwise per group.
  constexpr bool XPRE = P * MT <= 4;
  const uint32_t bias = bias_in_vgpr();

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
          else a[mt][s] = *reinterpret_cast<const f16x8*>(x + xrow[mt] * K + k0 + 8 * s);
        }
#pragma unroll
      for (int t = 0; t < RW; ++t) {
        const ZeroForms zf = zero_forms(zz[p][t]);
        f32x4 d[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) d[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 b = word_minus_zero(wv[p][t][s], bias, zf);
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
  float* red = reinterpret_cast<float*>(smem);
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
  const size_t lds = (size_t)(MT == 1 ? W : 1) * RW * 16 * MT * 16 * sizeof(float);  // the waves' partial tiles
  dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW))), block((unsigned)(W * kWave));
  auto xp = reinterpret_cast<const f16*>(x);
  auto pp = reinterpret_cast<const uint32_t*>(packed);
  auto sp = reinterpret_cast<const f16*>(scales);
  auto zp = reinterpret_cast<const uint8_t*>(zeros);
  auto yp = reinterpret_cast<f16*>(y);
  if (KernelPlan* p = active_plan())
    return plan_record(p, "skinny_kernel<%d,%d,%d> block=%u grid=%u", RW, P, MT, block.x, grid.x);
  skinny_kernel<RW, P, MT><<<grid, block, lds, st>>>(xp, pp, sp, zp, yp, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ring kernel, 2 <= M <= 16.  The register-staged kernel holds a batch's
// weight loads in registers until they land, so the bytes a CU keeps in flight
// are capped by its register file (about 64 KB at one block of eight waves per
// CU), and it streams the 70B-sized layers at a third of what the GEMV
// reaches.  Here weights and x fragments go from memory straight into LDS
// (global_load_lds_dwordx4, new in gfx950), which costs no registers while in
// flight: each wave owns a ring of S stages in LDS and keeps S - 1 of them
// loading while it computes on one.  A block's scales and zeros are staged in
// LDS once, before the first stage.
//
// A stage is one chunk of P consecutive groups for the block's RW tiles of 16
// rows (64 P bytes of each weight row) and for MX rows of x (256 P bytes
// each).  One DMA instruction fills 1 KB of LDS; each lane fetches the 16-byte
// piece (slot ^ swizzle(row)) of its row, so a row's reads stay contiguous in
// memory while the fragment reads of 16 rows (one piece each) hit 16 distinct
// bank groups.  3-bit codes (P = 1) take 48 bytes of a row per group: the
// rows go back to back as 16-byte pieces, and a lane reads the three words of
// its 32 channels (a 12-word row stride already spreads 16 rows over distinct
// banks).  Waves take chunks wave, wave + W, ....  Vector-memory
// operations complete in issue order, so one wait per stage, on the number of
// DMA instructions issued after the stage's own, says it has landed; the
// compiler tracks no LDS-DMA dependences, so these waits are explicit.  x rows
// past M hold row M - 1: MFMA output rows are independent and never stored.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_void;

// s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLds = 15 | (3 << 14) | (7 << 4);
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU

template <int P>
__device__ inline int ring_swizzle(int r) {
  return (r / (4 / P)) & (4 * P - 1);
}

template <int BITS, int RW, int P, int S, int MX>
__global__ __launch_bounds__(512) void ring_kernel(const f16* __restrict__ x, const uint32_t* __restrict__ packed,
                                                   const f16* __restrict__ scales, const uint8_t* __restrict__ zeros,
                                                   f16* __restrict__ y, int M, int N32, int K32, int W) {
  static_assert((P == 1 || P == 2) && S >= 2 && S <= 4 && MX % 4 == 0 && (MX <= 16 || MX % 16 == 0) && MX <= 64,
                "ring shape");
  constexpr int MT = MX > 16 ? MX / 16 : 1;  // 16-row x tiles; each weight operand feeds MT MFMAs
  static_assert(BITS == 4 || (BITS == 3 && P == 1), "4-bit, or 3-bit in one-group chunks");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int ROWB = 64 * P, RPI = 1024 / ROWB, SLOTS = 4 * P;
  // 4-bit: 16 rows x 64 P bytes per tile, NI instructions of 1 KB each; 3-bit: rows of
  // 48 bytes (three 16-byte pieces) back to back over the RW tiles, in NI instructions.
  constexpr int NI = BITS == 4 ? RW * (16 / RPI) : (48 * RW + 63) / 64;
  constexpr int TILE = BITS == 4 ? 16 * ROWB : 16 * 48;
  constexpr int XROWB = 256 * P, XRPI = 1024 / XROWB, NXI = MX / XRPI, XSLOTS = 16 * P;
  constexpr int WBYTES = NI * 1024;  // the weights of a stage, padded to whole instructions
  constexpr int STAGE = WBYTES + MX * XROWB;
  constexpr int NIS = NI + NXI;  // DMA instructions per stage
  const int64_t N = N32, K = K32, K8 = K / 8, G = K / kGroup, P2 = (G + 1) / 2, NC = (G + P - 1) / P;
  const int64_t RW3 = 3 * K / 32;  // 3-bit: words per row
  const int lane = threadIdx.x & 63, nl = lane & 15, kq = lane >> 4;
  // wave-uniform, so the chunk index, its clamps and the LDS destinations stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RW);
  const int T = (int)((NC + W - 1) / W);  // stages per wave; chunks past the last are reloaded, scaled by 0
  unsigned char* ring = smem + (size_t)wave * (S * STAGE);
  // the block's scales and zeros, staged once after the rings (each padded to whole KB)
  const int SCB = (int)(32 * RW * G), ZB = (int)(16 * RW * P2);
  f16* sl = reinterpret_cast<f16*>(smem + (size_t)W * S * STAGE);
  uint8_t* zl = reinterpret_cast<uint8_t*>(smem + (size_t)W * S * STAGE + ((SCB + 1023) & ~1023));
  const ScaleSwizzle ssw(G);  // the staged scales' layout

  // Weight DMA source of this lane per instruction, less the group's offset (4-bit:
  // row start + quarter, and the piece's group within the chunk in dgi; 3-bit: row
  // start + piece, for piece q * 64 + lane of the stage, clamped to the last).
  int64_t dsrc[NI];
  int dgi[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    if constexpr (BITS == 4) {
      const int t = q / (16 / RPI), qq = q % (16 / RPI);
      const int r = qq * RPI + lane / SLOTS, piece = (lane % SLOTS) ^ ring_swizzle<P>(r);
      dgi[q] = piece >> 2;
      const int64_t n = n0 + 16 * t + r;
      dsrc[q] = (n < N ? n : N - 1) * K8 + (piece & 3) * 4;  // tail rows reload the last row; never stored
    } else {
      const int pc = q * 64 + lane < 48 * RW ? q * 64 + lane : 48 * RW - 1;
      const int64_t n = n0 + pc / 3;
      dgi[q] = 0;
      dsrc[q] = (n < N ? n : N - 1) * RW3 + (pc % 3) * 4;
    }
  }
  // x DMA: LDS row r of a stage holds x row min(r, M - 1); piece slot ^ (r & 15) of it
  int64_t xsrc[NXI];
  int xgi[NXI];
#pragma unroll
  for (int q = 0; q < NXI; ++q) {
    const int r = q * XRPI + lane / XSLOTS, piece = (lane % XSLOTS) ^ (r & 15);
    xgi[q] = piece >> 4;
    xsrc[q] = (int64_t)(r < M ? r : M - 1) * K + (piece & 15) * 8;
  }

  f32x4 acc[RW][MT];
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int j) {
    int64_t c = (int64_t)j * W + wave;
    c = c < NC ? c : NC - 1;
    unsigned char* dst = ring + (j % S) * STAGE;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      int64_t g = c * P + dgi[q];
      g = g < G ? g : G - 1;
      __builtin_amdgcn_global_load_lds((global_void*)(packed + dsrc[q] + g * (BITS == 4 ? 16 : 12)),
                                       (lds_void*)(dst + q * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < NXI; ++q) {
      int64_t g = c * P + xgi[q];
      g = g < G ? g : G - 1;
      __builtin_amdgcn_global_load_lds((global_void*)(x + xsrc[q] + g * kGroup), (lds_void*)(dst + WBYTES + q * 1024), 16, 0,
                                       0);
    }
  };

  // A full block's rows are consecutive, so its scales and zeros are two contiguous
  // runs of whole 16-byte pieces: DMA them; a ragged last block copies them one by one.
  if (n0 + 16 * RW <= N) {
    const unsigned char* gs = reinterpret_cast<const unsigned char*>(scales) + n0 * G * 2;
    const unsigned char* gz = zeros + n0 * P2;
    for (int b = wave * kWave; b < SCB / 16; b += W * kWave) {
      const int v = b + lane < SCB / 16 ? b + lane : SCB / 16 - 1;  // lanes past the end land in the padding
      __builtin_amdgcn_global_load_lds((global_void*)(gs + ssw.piece_src(v) * 16),
                                       (lds_void*)(reinterpret_cast<unsigned char*>(sl) + b * 16), 16, 0, 0);
    }
    for (int b = wave * kWave; b < ZB / 16; b += W * kWave) {
      const int v = b + lane < ZB / 16 ? b + lane : ZB / 16 - 1;
      __builtin_amdgcn_global_load_lds((global_void*)(gz + v * 16), (lds_void*)(zl + b * 16), 16, 0, 0);
    }
  } else {
    for (int i = threadIdx.x; i < 16 * RW * G; i += W * kWave) {
      const int r = (int)(i / G);
      const int64_t n = n0 + r, g = i - (int64_t)r * G;
      sl[(int64_t)r * G + (g ^ ssw.xor_of(r))] = scales[(n < N ? n : N - 1) * G + g];
    }
    for (int i = threadIdx.x; i < ZB; i += W * kWave) {
      const int r = (int)(i / P2);
      const int64_t n = n0 + r;
      zl[i] = zeros[(n < N ? n : N - 1) * P2 + (i - (int64_t)r * P2)];
    }
  }
  for (int j = 0; j < S - 1 && j < T; ++j) issue(j);
  // the staged scales and zeros are read by every wave: all of this wave's loads land, then the barrier
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  int sxr[RW];  // scale xor of the lane's row in each weight tile
#pragma unroll
  for (int t = 0; t < RW; ++t) sxr[t] = ssw.xor_of(16 * t + nl);
  int xr[MT];  // LDS x row of the lane's A operand in x tile mt (rows past MX repeat the last)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xr[mt] = 16 * mt + nl < MX ? 16 * mt + nl : MX - 1;
  const uint32_t bias = bias_in_vgpr();
  for (int j = 0; j < T; ++j) {
    // the slot refilled here was read by the previous stage, whose LDS reads are done
    __builtin_amdgcn_s_waitcnt(kWaitLds);
    __builtin_amdgcn_sched_barrier(0);
    const int ahead = T - 1 - j;  // stages issued after this one
    if (ahead >= S - 1) {
      issue(j + S - 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 1) * NIS));
    } else if (S > 3 && ahead == 2) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NIS));
    } else if (S > 2 && ahead == 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(NIS));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t c = (int64_t)j * W + wave;  // past NC only in the last stage of some waves
    const unsigned char* src = ring + (j % S) * STAGE;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int64_t g = c * P + i;
      const bool live = g < G;
      const int gc = (int)(live ? g : G - 1);
      // Every LDS read of the chunk (x fragments, then each tile's codes, zero
      // byte and scale) is issued before the first use: one LDS round trip per
      // chunk rather than one per tile.  The scale is read unconditionally (gc is
      // clamped) and zeroed by a select for chunks past G.
      f16x8 a[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          a[mt][s] = *reinterpret_cast<const f16x8*>(src + WBYTES + xr[mt] * XROWB +
                                                     ((i * 16 + kq * 4 + s) ^ (xr[mt] & 15)) * 16);
      u32x4 wt[RW];
      uint32_t zt[RW];
      f16 st[RW];
#pragma unroll
      for (int t = 0; t < RW; ++t) {
        const int r = 16 * t + nl;
        if constexpr (BITS == 4) {
          wt[t] = *reinterpret_cast<const u32x4*>(src + t * TILE + nl * ROWB + ((i * 4 + kq) ^ ring_swizzle<P>(nl)) * 16);
        } else {
          // the three words of the lane's 32 channels (rows of 48 bytes: 16 rows on
          // distinct banks)
          const uint32_t* wp = reinterpret_cast<const uint32_t*>(src + r * 48 + kq * 12);
          wt[t] = u32x4{wp[0], wp[1], wp[2], 0u};
        }
        zt[t] = zl[r * P2 + (gc >> 1)];
        st[t] = sl[r * G + (gc ^ sxr[t])];
      }
#pragma unroll
      for (int t = 0; t < RW; ++t) {
        const ZeroForms zf = zero_forms((zt[t] >> (4 * (gc & 1))) & 0xFu);
        f32x4 d[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) d[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BITS == 4) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const f16x8 b = word_minus_zero(wt[t][s], bias, zf);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][s], b, d[mt], 0, 0, 0);
          }
        } else {
          // channel pair p of the chunk, as fp16 (1024 + code) pairs less (1024 + zero)
          const uint32_t w[3] = {wt[t][0], wt[t][1], wt[t][2]};
          f16x2 q[16];
#pragma unroll
          for (int pp = 0; pp < 15; ++pp)
            q[pp] = as_f16x2(((w[pp / 5] >> (3 * (pp % 5))) & 0x00070007u) | bias) - zf.zb1;
          q[15] = as_f16x2(((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) | ((w[2] >> 13) & 0x00040004u) |
                           bias) -
                  zf.zb1;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const f16x8 b = f16x8{q[4 * s].x,     q[4 * s].y,     q[4 * s + 1].x, q[4 * s + 1].y,
                                  q[4 * s + 2].x, q[4 * s + 2].y, q[4 * s + 3].x, q[4 * s + 3].y};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][s], b, d[mt], 0, 0, 0);
          }
        }
        const float scf = live ? (float)st[t] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[t][mt][rr] = fmaf(scf, d[mt][rr], acc[t][mt][rr]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // every wave's DMA has landed (the last stage waited for all); the rings become the
  // reduction buffer (W x RW x 16 MT x 16 fp32, within the rings): lane holds
  // y[m = 16 mt + 4 kq + r][n0 + 16 t + nl]
  constexpr int MR = 16 * MT;
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < RW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * kq + r;
        if (m < M) red[((wave * RW + t) * MR + m) * 16 + nl] = acc[t][mt][r];
      }
  __syncthreads();
  for (int i = threadIdx.x; i < RW * 16 * M; i += W * kWave) {
    const int t = i / (16 * M), rem = i - t * 16 * M, m = rem >> 4, nn = rem & 15;
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += red[((w * RW + t) * MR + m) * 16 + nn];
    const int64_t n = n0 + 16 * t + nn;
    if (n < N) y[(int64_t)m * N + n] = (f16)v;
  }
}

template <int BITS, int RW, int P, int S, int MX>
static size_t ring_lds_bytes(int W, int64_t K) {
  const int64_t G = K / kGroup;
  const size_t sc = (size_t)32 * RW * G, z = (size_t)16 * RW * ((G + 1) / 2);
  const size_t wbytes = BITS == 4 ? (size_t)RW * 1024 * P : (size_t)(48 * RW + 63) / 64 * 1024;
  return (size_t)W * S * (wbytes + MX * 256 * P) + ((sc + 1023) & ~(size_t)1023) + ((z + 1023) & ~(size_t)1023);
}

template <int P>
static int ring_waves(int max_waves, int64_t K) {
  const int64_t NC = (K / kGroup + P - 1) / P;
  return (int)(NC < max_waves ? NC : max_waves);
}

template <int BITS, int RW, int P, int S, int MX>
static hipError_t ring_launch(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                              int64_t N, int64_t K, int max_waves, hipStream_t st) {
  const int W = ring_waves<P>(max_waves, K);
  const size_t lds = ring_lds_bytes<BITS, RW, P, S, MX>(W, K);
  if (lds > kLdsBytes) return hipErrorInvalidValue;
  dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW))), block((unsigned)(W * kWave));
  if (KernelPlan* p = active_plan())
    return plan_record(p, "ring_kernel<%d,%d,%d,%d,%d> block=%u grid=%u", BITS, RW, P, S, MX, block.x, grid.x);
  ring_kernel<BITS, RW, P, S, MX><<<grid, block, lds, st>>>(
      reinterpret_cast<const f16*>(x), reinterpret_cast<const uint32_t*>(packed), reinterpret_cast<const f16*>(scales),
      reinterpret_cast<const uint8_t*>(zeros), reinterpret_cast<f16*>(y), (int)M, (int)N, (int)K, W);
  return hipGetLastError();
}

// Ring shape: one-group chunks in a two-stage ring (deeper rings cost blocks per
// CU and measured slower); 16-row tiles per wave and waves per block by layer
// shape, measured on the Llama-2 7B/70B decode shapes at M = 4, 8, 16.  The
// choice mostly sets how evenly the blocks fill 256 CUs: one tile and eight
// waves for M <= 4 and on layers up to 4096 wide; one tile and four waves on
// K <= 4096 (4096 x 11008 at M = 16: 11.6 us against 14.8) and on layers up
// to 16384 wide; two tiles and four waves on wider ones (8192 x 28672 at
// M = 16: 44 us against 58 with eight waves); two tiles and eight waves on
// the rest (8192 x 8192, 28672 x 8192).  Every block reads all of x (M rows x
// K), so for M > 4 wider blocks share it among more weight rows: on layers at
// least 16384 wide two tiles and four waves for K < 8192 (4096 x 22016 at
// M = 16: 18.7 us against 22.7 with one tile; at M = 8: 15.6 against 16.9) and
// four tiles and four waves for K >= 8192 (8192 x 28672: 38.0 us against 43.4
// at M = 16, 35.6 against 36.2 at M = 8); for M > 8 on the 70B q/k/v (8192 <
// N < 16384, K >= 8192) four tiles and eight waves (8192 x 10240: 20.9 us
// against 22.6; at M = 8 that shape is slower, 18.7 against 17.4, with only
// 160 blocks).
constexpr int kRingP = 1, kRingStages = 2;

struct RingShape {
  int rw, waves;
};

static RingShape ring_shape(int64_t M, int64_t N, int64_t K) {
  if (M > 4 && N >= 16384) return {K >= 8192 ? 4 : 2, 4};
  if (M > 8 && K >= 8192 && N > 8192) return {4, 8};
  if (M <= 4 || N <= 4096) return {1, 8};
  if (K <= 4096 || (N > 8192 && N < 16384)) return {1, 4};
  if (N >= 16384) return {2, 4};
  return {2, 8};
}

template <int BITS, int MX>
static bool ring_fits(const RingShape& r, int64_t K) {
  const int W = ring_waves<kRingP>(r.waves, K);
  if (r.rw == 1) return ring_lds_bytes<BITS, 1, kRingP, kRingStages, MX>(W, K) <= kLdsBytes;
  if (r.rw == 4) return ring_lds_bytes<BITS, 4, kRingP, kRingStages, MX>(W, K) <= kLdsBytes;
  return ring_lds_bytes<BITS, 2, kRingP, kRingStages, MX>(W, K) <= kLdsBytes;
}

template <int BITS, int MX>
static hipError_t ring_dispatch(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                                int64_t N, int64_t K, const RingShape& r, hipStream_t st) {
  if (r.rw == 1) return ring_launch<BITS, 1, kRingP, kRingStages, MX>(x, packed, scales, zeros, y, M, N, K, r.waves, st);
  if (r.rw == 4) return ring_launch<BITS, 4, kRingP, kRingStages, MX>(x, packed, scales, zeros, y, M, N, K, r.waves, st);
  return ring_launch<BITS, 2, kRingP, kRingStages, MX>(x, packed, scales, zeros, y, M, N, K, r.waves, st);
}

template <int BITS>
static bool ring_select(int64_t M, int64_t K, const RingShape& r, int* mx) {
  *mx = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
  if (M < 2 || M > 16) return false;
  return *mx == 4 ? ring_fits<BITS, 4>(r, K) : (*mx == 8 ? ring_fits<BITS, 8>(r, K) : ring_fits<BITS, 16>(r, K));
}

template <int BITS>
static hipError_t ring_run(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                           int64_t N, int64_t K, const RingShape& r, int mx, hipStream_t st) {
  if (mx == 4) return ring_dispatch<BITS, 4>(x, packed, scales, zeros, y, M, N, K, r, st);
  if (mx == 8) return ring_dispatch<BITS, 8>(x, packed, scales, zeros, y, M, N, K, r, st);
  if (mx == 32) return ring_dispatch<BITS, 32>(x, packed, scales, zeros, y, M, N, K, r, st);
  if (mx == 64) return ring_dispatch<BITS, 64>(x, packed, scales, zeros, y, M, N, K, r, st);
  return ring_dispatch<BITS, 16>(x, packed, scales, zeros, y, M, N, K, r, st);
}

// 17 <= M <= 64: two or four 16-row x tiles per stage, each weight operand
// feeding that many MFMAs.  Measured against the register-staged multi-row
// kernel and the pipelined GEMM at M = 24, 32, 48, 64 (us, ring / previous):
// 4096 x 4096 10.4-15.6 / 16.2-26.7; 11008 x 4096 18.2-29.6 / 32.3-56.6;
// 28672 x 8192 54-56 with two tiles per block at M <= 32 / 84-94, 109-123
// with one above / 118-143; 4096 x 11008 19.5-20.0 / 24.7-26.3 at M <= 32,
// but 33-38 / 28 above; 8192 x 28672 no better than the GEMM (66-135 / 67-71);
// 8192 x 10240 and 8192 x 12288 29.8-33.3 / 41.9-47.5 at M = 20-32 with one
// tile per block, 50.2-53.7 / 56.7-57.9 above with two; 6144 x 12288 26.2-27.2
// / 31.9-35.6 at M = 24-32, but 42.6-44.7 / 36.1-36.6 above; wider layers
// with K >= 8192 at M <= 32 with four tiles per block: 8192 x 28672 55.3-57.8
// / 66.4-68.1, 8192 x 16384 30.5-31.7 / 58.0-58.9 (two tiles: 65-67, 35-37);
// above M = 32 they stay on the GEMM (the best ring layout gains at most 4%
// there, and the layout that wins on one shape loses up to 40% on the other).
// On K <= 4096 layers up to M = 32, two or four tiles per block come within 3%
// of one (4096 x 11008, 4096 x 22016 at M = 20-32), so one it is.
// Waves per block: four.  {0, 0}: the layer goes to the other kernels.
static RingShape ring_mid_shape(int64_t M, int64_t N, int64_t K) {
  if (N <= 8192) return {K >= 16384 && M <= 32 ? 2 : 1, 4};
  if (M <= 32 && K <= 4096) return {1, 4};
  if (N <= 12288 && (M <= 32 ? K > 4096 : K >= 8192)) return {M > 32 ? 2 : 1, 4};
  if (M <= 32 && K >= 8192) return {4, 4};
  return {0, 0};
}

template <int BITS>
static bool ring_mid_select(int64_t M, int64_t K, const RingShape& r, int* mx) {
  if (M <= 16 || M > 64) return false;
  *mx = M <= 32 ? 32 : 64;
  return *mx == 32 ? ring_fits<BITS, 32>(r, K) : ring_fits<BITS, 64>(r, K);
}

// At 3 bits the alternative for M > 16 is the general-shape kernel (2-6x
// slower than the ring where both run: 28672 x 8192 at M = 24, 53 against
// 286 us), so the ring takes every layer there that the 3-bit pipelined GEMM
// does not.
static RingShape ring_mid_shape_bits(int64_t M, int64_t N, int64_t K, int bits) {
  const RingShape r = ring_mid_shape(M, N, K);
  if (r.rw == 0 && bits == 3) {  // two weight tiles per block above M = 32, as on 8192 x 10240
    const RingShape r2{2, 4};
    return M > 32 && ring_fits<3, 64>(r2, K) ? r2 : RingShape{1, 4};
  }
  return r;
}

// 3-bit codes, 32 < M <= 64 on a layer with no ring layout of its own: the
// pipelined GEMM where the layer is very wide or K is short (8192 x 28672 at
// M = 64: 71 against 135 us on the fallback ring layout; 4096 x 11008: 31
// against 38), the ring elsewhere (8192 x 10240 at M = 48: 55 against 60 us on
// the pipelined GEMM, and about even at M <= 32).
bool ring_mid_pipe_preferred(int64_t M, int64_t N, int64_t K) {
  return M > 32 && M <= 64 && ring_mid_shape(M, N, K).rw == 0 && (N > 12288 || K <= 4096);
}

bool ring_mid_supported(int64_t M, int64_t N, int64_t K, int bits) {
  const RingShape r = ring_mid_shape_bits(M, N, K, bits);
  int mx;
  if (r.rw == 0) return false;
  return bits == 3 ? ring_mid_select<3>(M, K, r, &mx) : ring_mid_select<4>(M, K, r, &mx);
}

hipError_t launch_ring_mid(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                           int64_t M, int64_t N, int64_t K, int bits, hipStream_t st) {
  const RingShape r = ring_mid_shape_bits(M, N, K, bits);
  int mx;
  if (r.rw == 0) return hipErrorInvalidValue;
  if (bits == 3) {
    if (!ring_mid_select<3>(M, K, r, &mx)) return hipErrorInvalidValue;
    return ring_run<3>(x, packed, scales, zeros, y, M, N, K, r, mx, st);
  }
  if (!ring_mid_select<4>(M, K, r, &mx)) return hipErrorInvalidValue;
  return ring_run<4>(x, packed, scales, zeros, y, M, N, K, r, mx, st);
}

// 3-bit codes, 2 <= M <= 16: the ring kernel with rows of 48 bytes, tile and
// wave shape as at 4 bits.
bool ring3_supported(int64_t M, int64_t N, int64_t K) {
  int mx;
  return ring_select<3>(M, K, ring_shape(M, N, K), &mx);
}

hipError_t launch_ring3(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                        int64_t N, int64_t K, hipStream_t st) {
  const RingShape r = ring_shape(M, N, K);
  int mx;
  if (!ring_select<3>(M, K, r, &mx)) return hipErrorInvalidValue;
  return ring_run<3>(x, packed, scales, zeros, y, M, N, K, r, mx, st);
}

// 17 <= M <= 64 where the ring declines: the register-staged kernel with M in
// up to four 16-row m-tiles (each unpacked weight operand feeds one MFMA per
// m-tile) on layers up to 8192 rows whose K leaves the ring no LDS beside the
// block's scales and zeros (K beyond ~130,000); every other such layer goes to
// the pipelined GEMM (or, past its LDS too, the general-shape kernel).
// Measured against the pipelined GEMM at M = 24..64 on layers up to 8192 rows,
// before the ring took them: 4096 x 4096 at 14-25 us against 24 us, 8192 x 8192
// at 27-46 us against 53 us, 28672 x 8192 at 81-139 us against 239 us.
bool gemv_wide_preferred(int64_t M, int64_t N, int64_t K) {
  (void)K;
  return M > 16 && M <= 64 && N <= 8192;
}

hipError_t launch_gemv_wide(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 16 || M > 64) return hipErrorInvalidValue;
  if (M <= 32) return skinny_launch<2, 1, 2>(x, packed, scales, zeros, y, M, N, K, st);
  if (M <= 48) return skinny_launch<2, 1, 3>(x, packed, scales, zeros, y, M, N, K, st);
  return skinny_launch<2, 1, 4>(x, packed, scales, zeros, y, M, N, K, st);
}

// M <= 16 beyond the GEMV's range runs on the ring kernel.  Where the ring
// declines (2 <= M <= 16 with K at least 16384 whose block scales and zeros
// leave the rings no LDS, and M = 1 beyond the GEMV's K = 32768) the
// register-staged kernel runs with two 16-row weight tiles per wave in batches
// of four groups (measured best on long K among its layouts).
hipError_t launch_gemv(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t st) {
  if (M < 1 || M > 16) return hipErrorInvalidValue;
  if (gemv_dot2_supported(M, K)) return launch_gemv_dot2(x, packed, scales, zeros, y, M, N, K, st);
  const RingShape r = ring_shape(M, N, K);
  int mx;
  if (ring_select<4>(M, K, r, &mx)) return ring_run<4>(x, packed, scales, zeros, y, M, N, K, r, mx, st);
  return skinny_launch<2, 4>(x, packed, scales, zeros, y, M, N, K, st);
}

}  // namespace awq
