// CPU oracle for AWQ's scale search, group-wise int4 / int3 quantizer and
// W4A16 product, in plain C++ (OpenMP over independent rows only).
//
// TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
// bench's CPU-baseline leg load this library (through oracle/cpp_oracle.py).
// It shares no code with the HIP library.
//
// Sources (titles of the pages the method is taken from):
//   [summary]  "AWQ: Activation-aware Weight Quantization for On-Device LLM
//              Compression and Acceleration", fdeinterviews.com/papers/awq,
//              cited by paragraph.
//   [abstract] OpenAlex record of the GetMobile article of the same title.
//
// Arithmetic.  The quantizer runs in IEEE fp32: every operation below is one
// fp32 operation rounded to nearest even (the file is compiled with
// -ffp-contract=off, so no multiply-add is fused, and without fast-math).
// Dequantization, the loss and the product run in fp64.  Sums over a row are
// formed in a fixed order and rows are combined in a fixed order, so results
// do not depend on the number of threads.
//
// Readings of points the pages leave open (listed with the design notes):
//   R1  "average activation magnitude" = mean over calibration rows of |x|,
//       formed exactly as an integer count of 2^-24.
//   R2  s = a^alpha (fp64 pow, rounded once to fp32), no normalisation or
//       clamp; a channel with a = 0 gets s = 1.
//   R3  min-max asymmetric uniform quantizer per group of `group` input
//       channels of one output row, range widened to include 0, step rounded
//       to fp16 (nearest even), integer zero point, codes rint(v / step) + z
//       with round-half-even and true division.
//   R4  objective: mean squared change of the layer's output on the
//       calibration rows, ||X E^T||^2 / (M N), E = w_hat / s - w.
//   R5  ties in the search go to the smallest alpha.
//   R6  keep-fp16 ablation: plain rounding (s = 1), then the kept channels'
//       weights restored exactly; the magnitude of a weight channel is the
//       mean of |w| over output rows.
//   R7  top channels: largest first, equal values by the lower index.
//   R11 the scaled input x / s is one fp32 division rounded to fp16.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------- fp16
// fp16 bit pattern -> fp32 value (exact: every fp16 value is an fp32 value).
float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 31u, m = h & 1023u;
  uint32_t bits;
  if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);  // inf / NaN
  } else if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {  // subnormal m * 2^-24: normalise
      int sh = 0;
      uint32_t mm = m;
      while (!(mm & 1024u)) {
        mm <<= 1;
        ++sh;
      }
      bits = sign | ((uint32_t)(113 - sh) << 23) | ((mm & 1023u) << 13);
    }
  } else {
    bits = sign | ((e + 112u) << 23) | (m << 13);
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

// fp32 -> fp16 bit pattern, round to nearest even, with integer operations
// only: overflow goes to infinity, values below half the smallest subnormal
// to zero; a NaN keeps its top 10 payload bits and becomes quiet.
uint16_t f32_to_f16(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const uint32_t ex = (x >> 23) & 255u, man = x & 0x7FFFFFu;
  if (ex == 255) return (uint16_t)(sign | 0x7C00u | (man ? (0x200u | (man >> 13)) : 0u));
  const int e = (int)ex - 127;        // unbiased exponent
  if (e > 15) return (uint16_t)(sign | 0x7C00u);  // at least 2^16: infinity
  if (ex == 0) return sign;           // fp32 zero or subnormal: far below 2^-25
  const uint32_t sig = man | 0x800000u;  // 24-bit significand, value sig * 2^(e - 23)
  // Normal fp16 (e >= -14): keep 11 bits, field (e + 14) << 10 plus the kept
  // value (whose implicit bit adds the 1 << 10).  Subnormal fp16: the value in
  // units of 2^-24 is sig * 2^(e + 1), so shift right by -(e + 1).
  const int shift = e >= -14 ? 13 : -1 - e;
  if (shift > 24) return sign;  // below 2^-25: rounds to zero
  const uint32_t base = e >= -14 ? (uint32_t)(e + 14) << 10 : 0u;
  const uint32_t kept = sig >> shift, rem = sig & ((1u << shift) - 1u), half = 1u << (shift - 1);
  const uint32_t r = kept + ((rem > half || (rem == half && (kept & 1u))) ? 1u : 0u);
  uint32_t h = base + r;  // a carry out of the 10-bit field bumps the exponent, up to infinity
  if (h >= 0x7C00u) h = 0x7C00u;
  return (uint16_t)(sign | h);
}

// Exact |x| of an fp16 value as a count of 2^-24 (below 2^40).
int64_t abs_units(uint16_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  if (e == 0) return m;
  return (int64_t)(1024u + m) << (e - 1);
}

// ---------------------------------------------------------------- quantizer
struct GroupQ {
  float lo, hi, step, sc;
  uint16_t sc16;
  float z;
};

// One group of V (fp32 values, count n): range, fp16 step, zero point, codes.
GroupQ quantize_group(const float* v, int n, float qmax, uint8_t* q) {
  GroupQ g;
  g.lo = 0.0f;
  g.hi = 0.0f;
  for (int i = 0; i < n; ++i) {
    g.lo = std::min(g.lo, v[i]);
    g.hi = std::max(g.hi, v[i]);
  }
  const float range = g.hi - g.lo;
  g.step = range / qmax;
  const float floor16 = 6.103515625e-05f;  // 2^-14, the smallest normal fp16
  if (g.step < floor16) g.step = floor16;
  g.sc16 = f32_to_f16(g.step);
  g.sc = f16_to_f32(g.sc16);
  const float zr = std::nearbyint(-g.lo / g.sc);
  g.z = std::min(std::max(zr, 0.0f), qmax);
  for (int i = 0; i < n; ++i) {
    const float t = std::nearbyint(v[i] / g.sc) + g.z;
    q[i] = (uint8_t)std::min(std::max(t, 0.0f), qmax);
  }
  return g;
}

double dequant(uint8_t q, uint8_t z, uint16_t sc16) {
  return ((double)q - (double)z) * (double)f16_to_f32(sc16);
}

}  // namespace

extern "C" {

uint16_t oracle_f32_to_f16(float f) { return f32_to_f16(f); }
float oracle_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

// a[k] = (1/M) sum_t |X[t][k]|, the sum exact ([summary] paragraph 3: each
// channel's average activation magnitude).
void oracle_channel_mean_abs(const uint16_t* X, int64_t M, int64_t K, double* a) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k) {
    int64_t s = 0;
    for (int64_t t = 0; t < M; ++t) s += abs_units(X[t * K + k]);
    a[k] = (double)s * 0x1p-24 / (double)M;  // s < 2^63 for M < 2^23
  }
}

// s[k] = fp32(a_k ^ alpha), 1 where a_k = 0 ([summary] paragraph 3).
void oracle_scales_for_alpha(const double* a, int64_t K, float alpha, float* s) {
  for (int64_t k = 0; k < K; ++k) s[k] = a[k] == 0.0 ? 1.0f : (float)std::pow(a[k], (double)alpha);
}

// V[n][k] = fp32(W[n][k]) * s[k] (s may be NULL: V = W).
void oracle_scale_weights(const uint16_t* W, const float* s, int64_t N, int64_t K, float* V) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) V[n * K + k] = s ? f16_to_f32(W[n * K + k]) * s[k] : f16_to_f32(W[n * K + k]);
}

// Group-wise quantization of V [N][K]: codes q [N][K], zero points z and fp16
// steps sc16 [N][K / group].
void oracle_quantize_groups(const float* V, int64_t N, int64_t K, int32_t group, int32_t bits, uint8_t* q,
                            uint8_t* z, uint16_t* sc16) {
  const float qmax = (float)((1 << bits) - 1);
  const int64_t G = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < G; ++j) {
      const GroupQ g = quantize_group(V + n * K + j * group, group, qmax, q + n * K + j * group);
      z[n * G + j] = (uint8_t)g.z;
      sc16[n * G + j] = g.sc16;
    }
}

// What[n][k] = (q - z) * sc in fp64 (exact).
void oracle_dequantize(const uint8_t* q, const uint8_t* z, const uint16_t* sc16, int64_t N, int64_t K, int32_t group,
                       double* What) {
  const int64_t G = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) What[n * K + k] = dequant(q[n * K + k], z[n * G + k / group], sc16[n * G + k / group]);
}

// E[n][k] = What[n][k] / s[k] - w[n][k] in fp64 (s may be NULL: s = 1).
void oracle_weight_error(const uint16_t* W, const uint8_t* q, const uint8_t* z, const uint16_t* sc16, const float* s,
                         int64_t N, int64_t K, int32_t group, double* E) {
  const int64_t G = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const double wh = dequant(q[n * K + k], z[n * G + k / group], sc16[n * G + k / group]);
      const double sd = s ? (double)s[k] : 1.0;
      E[n * K + k] = wh / sd - (double)f16_to_f32(W[n * K + k]);
    }
}

// The loops below take a few output rows at a time through a pass over the
// shared operand, so it is read from memory once per few rows rather than per
// row; every output still sums over k in increasing order.
constexpr int64_t kRowBlock = 8;

// Direct form: (1/(M N)) sum_t sum_n (sum_k X[t][k] E[n][k])^2.  Y[t][.]
// accumulates over k in order (vectorisable across n).
double oracle_output_mse(const uint16_t* X, int64_t M, int64_t K, const double* E, int64_t N) {
  std::vector<double> ET((size_t)K * (size_t)N);  // E transposed: ET[k][n]
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) ET[(size_t)k * N + n] = E[n * K + k];
  const int64_t nblk = (M + kRowBlock - 1) / kRowBlock;
  std::vector<double> row_sum((size_t)M);
#pragma omp parallel
  {
    std::vector<double> y((size_t)(kRowBlock * N));
#pragma omp for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
      const int64_t t0 = b * kRowBlock, t1 = std::min(M, t0 + kRowBlock);
      std::fill(y.begin(), y.end(), 0.0);
      for (int64_t k = 0; k < K; ++k) {
        const double* e = ET.data() + (size_t)k * N;
        for (int64_t t = t0; t < t1; ++t) {
          const double xv = (double)f16_to_f32(X[t * K + k]);
          double* yt = y.data() + (t - t0) * N;
          for (int64_t n = 0; n < N; ++n) yt[n] += xv * e[n];
        }
      }
      for (int64_t t = t0; t < t1; ++t) {
        const double* yt = y.data() + (t - t0) * N;
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s += yt[n] * yt[n];
        row_sum[t] = s;
      }
    }
  }
  double total = 0.0;
  for (int64_t t = 0; t < M; ++t) total += row_sum[t];
  return total / ((double)M * (double)N);
}

// G = X^T X in fp64, [K][K]: G[i][j] = sum_t X[t][i] X[t][j], over t in order.
void oracle_gram(const uint16_t* X, int64_t M, int64_t K, double* G) {
  std::vector<float> Xf((size_t)M * (size_t)K);  // fp16 values are exact in fp32
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M * K; ++i) Xf[i] = f16_to_f32(X[i]);
  const int64_t blk = 4 * kRowBlock, nblk = (K + blk - 1) / blk;
#pragma omp parallel for schedule(dynamic)
  for (int64_t b = 0; b < nblk; ++b) {
    const int64_t i0 = b * blk, i1 = std::min(K, i0 + blk);
    for (int64_t i = i0; i < i1; ++i)
      for (int64_t j = 0; j < K; ++j) G[i * K + j] = 0.0;
    for (int64_t t = 0; t < M; ++t) {
      const float* xr = Xf.data() + (size_t)t * K;
      for (int64_t i = i0; i < i1; ++i) {
        const double xi = (double)xr[i];
        double* g = G + i * K;
        for (int64_t j = 0; j < K; ++j) g[j] += xi * (double)xr[j];
      }
    }
  }
}

// Gram form of the same loss: (1/(M N)) sum_n E_n G E_n^T, the product
// T_n = E_n G summed over k in order.
double oracle_output_mse_gram(const double* G, int64_t K, const double* E, int64_t N, int64_t M) {
  const int64_t blk = 2 * kRowBlock, nblk = (N + blk - 1) / blk;
  std::vector<double> row_sum((size_t)N);
#pragma omp parallel
  {
    std::vector<double> t((size_t)(blk * K));
#pragma omp for schedule(dynamic)
    for (int64_t b = 0; b < nblk; ++b) {
      const int64_t n0 = b * blk, n1 = std::min(N, n0 + blk);
      std::fill(t.begin(), t.end(), 0.0);
      for (int64_t k = 0; k < K; ++k) {
        const double* g = G + k * K;
        for (int64_t n = n0; n < n1; ++n) {
          const double ek = E[n * K + k];
          double* tn = t.data() + (n - n0) * K;
          for (int64_t j = 0; j < K; ++j) tn[j] += ek * g[j];
        }
      }
      for (int64_t n = n0; n < n1; ++n) {
        const double* tn = t.data() + (n - n0) * K;
        const double* e = E + n * K;
        double s = 0.0;
        for (int64_t j = 0; j < K; ++j) s += tn[j] * e[j];
        row_sum[n] = s;
      }
    }
  }
  double total = 0.0;
  for (int64_t n = 0; n < N; ++n) total += row_sum[n];
  return total / ((double)M * (double)N);
}

// The scale search of [summary] paragraph 3 for one layer: for every alpha,
// s = a^alpha, quantize W diag(s), loss of w_hat / s on X; alpha* = the first
// smallest loss; outputs at alpha*.  use_gram: -1 picks the Gram form when
// M > K, 0 / 1 force the direct / Gram form.
void oracle_search(const uint16_t* W, const uint16_t* X, int64_t N, int64_t K, int64_t M, int32_t group, int32_t bits,
                   const float* alphas, int32_t n_alpha, int32_t use_gram, int32_t* best, double* losses, double* a,
                   uint8_t* q, uint8_t* z, uint16_t* sc16, float* s) {
  const bool gram = use_gram < 0 ? M > K : use_gram != 0;
  oracle_channel_mean_abs(X, M, K, a);
  std::vector<double> G;
  if (gram) {
    G.resize((size_t)K * (size_t)K);
    oracle_gram(X, M, K, G.data());
  }
  std::vector<float> V((size_t)N * (size_t)K), si((size_t)K);
  std::vector<double> E((size_t)N * (size_t)K);
  for (int32_t i = 0; i < n_alpha; ++i) {
    oracle_scales_for_alpha(a, K, alphas[i], si.data());
    oracle_scale_weights(W, si.data(), N, K, V.data());
    oracle_quantize_groups(V.data(), N, K, group, bits, q, z, sc16);
    oracle_weight_error(W, q, z, sc16, si.data(), N, K, group, E.data());
    losses[i] = gram ? oracle_output_mse_gram(G.data(), K, E.data(), N, M) : oracle_output_mse(X, M, K, E.data(), N);
  }
  int32_t b = 0;
  for (int32_t i = 1; i < n_alpha; ++i)
    if (losses[i] < losses[b]) b = i;
  *best = b;
  oracle_scales_for_alpha(a, K, alphas[b], s);
  oracle_scale_weights(W, s, N, K, V.data());
  oracle_quantize_groups(V.data(), N, K, group, bits, q, z, sc16);
}

// y[m][n] = sum_k x[m][k] (q[n][k] - z) sc in fp64 (x already divided by s).
void oracle_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q, const uint8_t* z, const uint16_t* sc16,
                 int64_t N, int32_t group, double* y) {
  const int64_t G = K / group;
#pragma omp parallel
  {
    std::vector<double> wrow((size_t)K);
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) wrow[k] = dequant(q[n * K + k], z[n * G + k / group], sc16[n * G + k / group]);
      for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += (double)f16_to_f32(xr[k]) * wrow[k];
        y[m * N + n] = acc;
      }
    }
  }
}

// xs = fp16(fp32(x) / s): one fp32 division per value, rounded to fp16 ([summary]
// paragraph 3: the input of a scaled channel is divided by s; reading R11).
void oracle_scaled_input(const uint16_t* x, int64_t M, int64_t K, const float* s, uint16_t* xs) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) xs[m * K + k] = f32_to_f16(f16_to_f32(x[m * K + k]) / s[k]);
}

// The n_keep largest entries of v, largest first, equal values by the lower index.
void oracle_top_channels(const double* v, int64_t K, int32_t n_keep, int32_t* out) {
  std::vector<int32_t> idx((size_t)K);
  for (int64_t k = 0; k < K; ++k) idx[k] = (int32_t)k;
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t i, int32_t j) { return v[i] > v[j]; });
  for (int32_t r = 0; r < n_keep; ++r) out[r] = idx[r];
}

// E = w_hat - w of plain rounding (s = 1) with the kept channels' columns
// exact ([summary] paragraph 2; reading R6).
void oracle_keep_fp16_error(const uint16_t* W, int64_t N, int64_t K, const int32_t* keep, int32_t n_keep,
                            int32_t group, int32_t bits, double* E) {
  std::vector<float> V((size_t)N * (size_t)K);
  std::vector<uint8_t> q((size_t)N * (size_t)K), z((size_t)N * (size_t)(K / group));
  std::vector<uint16_t> sc((size_t)N * (size_t)(K / group));
  oracle_scale_weights(W, nullptr, N, K, V.data());
  oracle_quantize_groups(V.data(), N, K, group, bits, q.data(), z.data(), sc.data());
  oracle_weight_error(W, q.data(), z.data(), sc.data(), nullptr, N, K, group, E);
  for (int32_t i = 0; i < n_keep; ++i) {
    const int64_t k = keep[i];
    if (k < 0 || k >= K) continue;
    for (int64_t n = 0; n < N; ++n) E[n * K + k] = 0.0;
  }
}

// Output MSE on X of plain rounding with n_keep channels kept in fp16: none,
// chosen by activation magnitude, by weight magnitude, and random_keep.
void oracle_keep_fp16_ablation(const uint16_t* W, const uint16_t* X, int64_t N, int64_t K, int64_t M, int32_t n_keep,
                               const int32_t* random_keep, int32_t group, int32_t bits, int32_t use_gram,
                               double* losses, int32_t* keep_act, int32_t* keep_wt, double* a, double* b) {
  const bool gram = use_gram < 0 ? M > K : use_gram != 0;
  oracle_channel_mean_abs(X, M, K, a);
  oracle_channel_mean_abs(W, N, K, b);  // mean over output rows of |w|: the same reduction
  oracle_top_channels(a, K, n_keep, keep_act);
  oracle_top_channels(b, K, n_keep, keep_wt);
  std::vector<double> G;
  if (gram) {
    G.resize((size_t)K * (size_t)K);
    oracle_gram(X, M, K, G.data());
  }
  std::vector<double> E((size_t)N * (size_t)K);
  const int32_t* sets[4] = {nullptr, keep_act, keep_wt, random_keep};
  for (int i = 0; i < 4; ++i) {
    oracle_keep_fp16_error(W, N, K, sets[i], i == 0 ? 0 : n_keep, group, bits, E.data());
    losses[i] = gram ? oracle_output_mse_gram(G.data(), K, E.data(), N, M) : oracle_output_mse(X, M, K, E.data(), N);
  }
}

}  // extern "C"
