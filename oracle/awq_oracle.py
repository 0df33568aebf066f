"""CPU oracle for AWQ's scale search, group-wise int4 quantizer and W4A16 product.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP path.

Sources (titles of the pages the method is taken from):
  [summary]  "AWQ: Activation-aware Weight Quantization for On-Device LLM
             Compression and Acceleration", fdeinterviews.com/papers/awq,
             cited by paragraph (P1..P10).
  [abstract] OpenAlex record of the GetMobile article of the same title
             (abstract).
  [glossary] "AWQ", dataterminology.com/term/awq (DESCRIPTION, TOP QUESTIONS).

Precision: the quantizer runs in IEEE float32 (numpy float32 ops round to
nearest-even and are never fused), dequantization, the loss and the product run
in float64.  Library primitives used as single steps: numpy matmul (BLAS) for
X @ E^T, X^T @ X, E @ G and x @ W^T; numpy's float32 -> float16 cast for the
round-to-nearest-even fp16 scale.

Readings of points the pages leave open (each is also listed in the design
notes of the repository):
  R1  "average activation magnitude" = mean over calibration rows of |x|.
  R2  s = a ** alpha with no normalisation and no clamp; a channel with a = 0
      gets s = 1.
  R3  the quantizer is min-max asymmetric uniform int4 per group of `group`
      consecutive input channels of one output row, with the range widened to
      include 0, fp16 scale, integer zero point, round-half-to-even, codes
      computed as rint(v / scale) + z with the fp16-rounded scale.
  R4  the search objective is the mean squared error of the layer's output on
      the calibration rows, against the unquantized layer.
  R5  ties in the search are broken towards the smallest alpha.
  R6  keep-fp16 ablation: the whole weight is rounded group-wise as usual (s = 1) and the
      kept channels' weights are then restored exactly; they are not removed from their
      groups' ranges, so every selection rule shares the same steps and codes.  The weight
      magnitude of an input channel is the mean of |w| over the output rows.
  R7  top channels: largest value first, equal values ordered by the lower index.
  R11 the scaled input x / s is one float32 division per value, rounded once to fp16.
"""
from __future__ import annotations

import numpy as np

# Smallest normal fp16 value; floor of a group's step so that a constant group
# still has a finite, non-zero fp16 scale.
SCALE_FLOOR = np.float32(2.0 ** -14)


def alpha_grid(n: int = 20) -> np.ndarray:
    """The search grid alpha_i = i / n, i = 0..n-1, as float32 ([summary] P3: grid search over alpha)."""
    return (np.arange(n, dtype=np.float32) / np.float32(n)).astype(np.float32)


# --------------------------------------------------------------------------- A1
def channel_mean_abs(X: np.ndarray) -> np.ndarray:
    """a_k = mean over rows t of |X[t, k]|, in float64 ([summary] P3: each channel's
    average activation magnitude; reading R1).

    Every finite fp16 |x| is an integer multiple of 2**-24, so the column sums
    are formed exactly as int64 counts of 2**-24 and only the final mean is
    rounded: a_k = float64(S_k) * 2**-24 / M.
    """
    X = np.asarray(X)
    assert X.dtype == np.float16 and X.ndim == 2
    M, K = X.shape
    S = np.zeros(K, dtype=np.int64)
    for r0 in range(0, M, 4096):  # row blocks only bound memory; integer sums are exact
        units = (np.abs(X[r0:r0 + 4096]).astype(np.float64) * 2.0 ** 24).astype(np.int64)
        S += units.sum(axis=0, dtype=np.int64)
    return S.astype(np.float64) * 2.0 ** -24 / np.float64(M)


# --------------------------------------------------------------------------- A3
def scales_for_alpha(a: np.ndarray, alpha) -> np.ndarray:
    """s_k = a_k ** alpha, evaluated in float64 and rounded to float32; s_k = 1 where
    a_k = 0 ([summary] P3: s from the average magnitude raised to a power alpha;
    reading R2)."""
    a = np.asarray(a, dtype=np.float64)
    al = np.float64(np.float32(alpha))
    s = np.power(a, al).astype(np.float32)
    s[a == 0.0] = np.float32(1.0)
    return s


def scale_weights(W: np.ndarray, s: np.ndarray) -> np.ndarray:
    """v[n, k] = float32(w[n, k]) * s[k] in float32: input channel k of the weight
    is multiplied by s_k ([summary] P3: multiply a weight channel by s)."""
    return np.asarray(W).astype(np.float32) * np.asarray(s, dtype=np.float32)[None, :]


# --------------------------------------------------------------------------- A4
def quantize_groups(V: np.ndarray, group: int = 128, bits: int = 4):
    """Group-wise asymmetric uniform quantization of V [N][K] (float32) (reading R3).

    For each output row n and group j (input channels group*j .. group*j+group-1):
        lo = min(0, min v),  hi = max(0, max v)             (float32)
        step = max((hi - lo) / (2**bits - 1), 2**-14)        (float32)
        sc = fp16(step)   (round to nearest even)            -> returned scale
        z  = clamp(rint(-lo / sc), 0, 2**bits - 1)
        q  = clamp(rint(v / sc) + z, 0, 2**bits - 1)
    Returns (q uint8 [N][K], z uint8 [N][K/group], sc float16 [N][K/group]).
    """
    V = np.asarray(V, dtype=np.float32)
    N, K = V.shape
    assert K % group == 0
    qmax = np.float32(2 ** bits - 1)
    Vg = V.reshape(N, K // group, group)
    lo = np.minimum(Vg.min(axis=2), np.float32(0.0))
    hi = np.maximum(Vg.max(axis=2), np.float32(0.0))
    step = np.maximum((hi - lo) / qmax, SCALE_FLOOR)
    sc16 = step.astype(np.float16)
    sc = sc16.astype(np.float32)
    z = np.clip(np.rint(-lo / sc), np.float32(0.0), qmax)
    q = np.clip(np.rint(Vg / sc[:, :, None]) + z[:, :, None], np.float32(0.0), qmax)
    return q.reshape(N, K).astype(np.uint8), z.astype(np.uint8), sc16


# --------------------------------------------------------------------------- A6/A7
def dequantize(q: np.ndarray, z: np.ndarray, sc16: np.ndarray, group: int = 128) -> np.ndarray:
    """w_hat[n, k] = (q[n, k] - z[n, j]) * sc[n, j] in float64 (exact), j = k // group."""
    N, K = q.shape
    zz = np.repeat(np.asarray(z, dtype=np.float64), group, axis=1)
    ss = np.repeat(np.asarray(sc16).astype(np.float64), group, axis=1)
    return (q.astype(np.float64) - zz) * ss


def effective_weight(q, z, sc16, s, group: int = 128) -> np.ndarray:
    """The layer the quantized model computes on unscaled inputs: w_hat / s along k
    ([summary] P3: divide the channel's input by s), float64."""
    return dequantize(q, z, sc16, group) / np.asarray(s, dtype=np.float32).astype(np.float64)[None, :]


def weight_error(W, q, z, sc16, s, group: int = 128) -> np.ndarray:
    """E = w_hat / s - w in float64."""
    return effective_weight(q, z, sc16, s, group) - np.asarray(W).astype(np.float64)


# --------------------------------------------------------------------------- A5
def output_mse(X: np.ndarray, E: np.ndarray) -> float:
    """L = ||X E^T||_F^2 / (M N): mean squared change of the layer's output over the
    calibration rows (reading R4), direct form."""
    X = np.asarray(X).astype(np.float64)
    D = X @ np.asarray(E, dtype=np.float64).T
    M, N = D.shape
    return float(np.sum(D * D) / (np.float64(M) * np.float64(N)))


def gram(X: np.ndarray) -> np.ndarray:
    """G = X^T X in float64."""
    X = np.asarray(X).astype(np.float64)
    return X.T @ X


def output_mse_gram(G: np.ndarray, E: np.ndarray, M: int) -> float:
    """The same L through the identity ||X E^T||^2 = sum_n E_n G E_n^T, G = X^T X."""
    E = np.asarray(E, dtype=np.float64)
    N = E.shape[0]
    return float(np.sum((E @ G) * E) / (np.float64(M) * np.float64(N)))


# --------------------------------------------------------------------------- A1..A6
def quantize_at(W, a, alpha, group: int = 128, bits: int = 4):
    """Scale by s(alpha), quantize; returns (q, z, sc16, s)."""
    s = scales_for_alpha(a, alpha)
    q, z, sc16 = quantize_groups(scale_weights(W, s), group, bits)
    return q, z, sc16, s


def search(W: np.ndarray, X: np.ndarray, group: int = 128, alphas=None, bits: int = 4,
           use_gram: bool | None = None) -> dict:
    """AWQ scale search for one linear layer ([summary] P3; [abstract]).

    For every alpha on the grid: s = a**alpha, quantize W diag(s), measure the
    output MSE of the effective weight (w_hat / s) on X.  alpha* is the first
    index of the smallest loss (reading R5).  The direct form of the loss is the
    definition; when M > K the Gram identity gives the same number with fewer
    flops (use_gram=None picks it then).
    """
    W = np.asarray(W)
    X = np.asarray(X)
    assert W.dtype == np.float16 and X.dtype == np.float16
    N, K = W.shape
    M = X.shape[0]
    assert X.shape[1] == K
    if alphas is None:
        alphas = alpha_grid(20)
    alphas = np.asarray(alphas, dtype=np.float32)
    if use_gram is None:
        use_gram = M > K
    a = channel_mean_abs(X)
    G = gram(X) if use_gram else None
    losses = np.zeros(len(alphas), dtype=np.float64)
    for i, al in enumerate(alphas):
        q, z, sc16, s = quantize_at(W, a, al, group, bits)
        E = weight_error(W, q, z, sc16, s, group)
        losses[i] = output_mse_gram(G, E, M) if use_gram else output_mse(X, E)
    best = 0
    for i in range(1, len(losses)):
        if losses[i] < losses[best]:
            best = i
    q, z, sc16, s = quantize_at(W, a, alphas[best], group, bits)
    return dict(alpha_index=best, alpha=float(alphas[best]), losses=losses, a=a,
                q=q, z=z, scales=sc16, s=s)


# --------------------------------------------------------------------------- keep-fp16 ablation
def top_channels(v: np.ndarray, n_keep: int) -> np.ndarray:
    """Indices of the n_keep largest entries of v, largest first; equal values are ordered
    by the lower index (reading R7)."""
    v = np.asarray(v, dtype=np.float64)
    order = sorted(range(v.shape[0]), key=lambda k: (-v[k], k))
    return np.array(order[:n_keep], dtype=np.int32)


def keep_fp16_error(W: np.ndarray, keep, group: int = 128, bits: int = 4) -> np.ndarray:
    """E = w_hat - w (float64) of plain group-wise rounding (s = 1), with the columns of the
    kept input channels exact ([summary] P2: a few channels stay in 16-bit while the rest
    are rounded).  The kept channels stay in their groups' ranges (reading R6)."""
    q, z, sc16 = quantize_groups(np.asarray(W).astype(np.float32), group, bits)
    E = dequantize(q, z, sc16, group) - np.asarray(W).astype(np.float64)
    E[:, np.asarray(keep, dtype=np.int64)] = 0.0
    return E


def keep_fp16_ablation(W: np.ndarray, X: np.ndarray, n_keep: int, random_keep, group: int = 128,
                       bits: int = 4, use_gram: bool | None = None) -> dict:
    """Output MSE on X of plain rounding with n_keep input channels kept in fp16, for the
    channels chosen by activation magnitude (largest mean |x|), by weight magnitude (largest
    mean |w| over output rows) and by the caller's random choice, next to keeping none
    ([summary] P2).  Losses in the order none, activation, weight, random."""
    W = np.asarray(W)
    X = np.asarray(X)
    M, K = X.shape
    if use_gram is None:
        use_gram = M > K
    a = channel_mean_abs(X)
    b = channel_mean_abs(W)  # mean over output rows of |w| per input channel: the same reduction
    sets = [np.zeros(0, np.int32), top_channels(a, n_keep), top_channels(b, n_keep),
            np.asarray(random_keep, dtype=np.int32)]
    G = gram(X) if use_gram else None
    losses = np.zeros(4, dtype=np.float64)
    for i, keep in enumerate(sets):
        E = keep_fp16_error(W, keep, group, bits)
        losses[i] = output_mse_gram(G, E, M) if use_gram else output_mse(X, E)
    return dict(losses=losses, keep_activation=sets[1], keep_weight=sets[2], a=a, b=b)


# --------------------------------------------------------------------------- NEXT-2
def scaled_input(x: np.ndarray, s) -> np.ndarray:
    """The fp16 input the W4A16 product takes: each channel of x divided by its s
    ([summary] P3: a channel scaled up by s in the weight has its input divided by s),
    as one float32 division rounded once to fp16 (reading R11)."""
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    return (x32 / np.asarray(s, dtype=np.float32)[None, :]).astype(np.float16)


# --------------------------------------------------------------------------- A8/A9
def gemm(x: np.ndarray, q, z, sc16, group: int = 128) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * (q[n, k] - z[n, k // group]) * sc[n, k // group], float64.

    x is the fp16 input already divided by s (the scale is folded into the
    input, [summary] P3), so this is the product the W4A16 kernels compute.
    """
    x = np.asarray(x)
    return x.astype(np.float64) @ dequantize(q, z, sc16, group).T
