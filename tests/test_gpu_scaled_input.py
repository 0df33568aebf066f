"""GPU parity of the input side of the per-channel scaling against the oracle.

awq_inverse_scale is IEEE fp32 division, checked bit for bit against numpy's; awq_scale_input
is one fp32 product rounded once to fp16, checked bit for bit against the same two numpy
operations, and against the oracle's x / s (one fp32 division rounded once), from which it
may differ only by one fp16 ulp on a few values.  awq_gemm_scaled must equal awq_gemm_bits
on awq_scale_input's output bit for bit (fused into the GEMV's x load at 4 bits, M <= 2 and N K <= 2^24,
through the workspace otherwise), and the oracle's product on x / s to the usual bars
(relative Frobenius error <= 1e-3, max |dy| <= 1e-2 max |y_ref|)."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16
from layout import assert_y_close
from test_gpu_parity import _random_packed, dev, host, note
from test_gpu_three_bit import _random_packed3

pytestmark = pytest.mark.gpu


def _scales(K, seed):
    """A layer's s: a^0.5 of a lognormal channel-magnitude profile (the search's range)."""
    g = np.random.default_rng(seed)
    a = np.exp(g.normal(0.0, 0.8, K))
    a[g.choice(K, max(1, K // 100), replace=False)] *= 20.0
    return oracle.scales_for_alpha(a, 0.5)


def test_inverse_scale_is_ieee_division():
    note("inverse scale")
    s = _scales(11008, 1)
    s[:4] = [1.0, 3.0, 0.1, 7.0]
    inv = host(awq.awq_inverse_scale(dev(s)))
    assert np.array_equal(inv.view(np.uint32), (np.float32(1.0) / s).view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 4096), (2, 11008), (37, 1024), (5, 8)])
def test_scale_input_bits(M, K):
    note(f"scale input M={M} K={K}")
    s = _scales(K, 2 + K)
    x = activations_fp16(M, K, seed=3 + M)
    inv = np.float32(1.0) / s
    xs = host(awq.awq_scale_input(dev(x), dev(inv)))
    want = (x.astype(np.float32) * inv[None, :]).astype(np.float16)
    assert np.array_equal(xs.view(np.uint16), want.view(np.uint16))
    ref = oracle.scaled_input(x, s)
    diff = xs.astype(np.float64) != ref.astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(xs.astype(np.float64) - ref.astype(np.float64)) <= ulp)
    assert diff.mean() <= 0.01, diff.mean()


@pytest.mark.parametrize("M,N,K,bits", [
    (1, 4096, 4096, 4), (2, 4096, 4096, 4), (1, 1000, 11008, 4), (2, 515, 2176, 4),  # fused GEMV
    (1, 11008, 4096, 4), (2, 4100, 4096, 4),                                           # larger: two launches
    (2, 300, 16384, 4),                                                                # M = 2, long rows
    (3, 700, 1024, 4), (16, 257, 2048, 4), (100, 300, 1024, 4),                        # workspace path
    (1, 600, 4096, 3), (7, 300, 1024, 3), (100, 300, 1024, 3),                         # 3-bit
])
def test_gemm_scaled_parity(M, N, K, bits):
    note(f"gemm scaled M={M} N={N} K={K} bits={bits}")
    seed = M + N + K + bits
    q, z, sc, p, scd, zd = (_random_packed if bits == 4 else _random_packed3)(N, K, seed=seed)
    s = _scales(K, seed + 1)
    x = activations_fp16(M, K, seed=seed + 2)
    inv = awq.awq_inverse_scale(dev(s))
    fused = bits == 4 and (M == 1 or (M == 2 and K < 16384)) and N * K <= 1 << 24
    assert (awq.awq_gemm_scaled_workspace_bytes(M, N, K, bits) == 0) == fused
    y = host(awq.awq_gemm_scaled(dev(x), inv, p, scd, zd, bits=bits))
    xs = awq.awq_scale_input(dev(x), inv)
    y2 = host(awq.awq_gemm(xs, p, scd, zd, bits=bits))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), f"M={M} N={N} K={K} bits={bits}"
    assert_y_close(y, oracle.gemm(oracle.scaled_input(x, s), q, z, sc), f"M={M} N={N} K={K} bits={bits}")


def test_gemm_scaled_recovers_unscaled_layer():
    """Quantize W diag(s) with the library, then run the unscaled x through awq_gemm_scaled:
    the result is the layer x W^T up to the quantization error (compared with the oracle's
    effective weight w_hat / s on the same codes)."""
    note("gemm scaled end to end")
    from gen import normal_fp16
    N, K = 512, 4096
    W = normal_fp16((N, K), 0.02, seed=41)
    s = _scales(K, 42)
    p, scd, zd = awq.awq_pack(dev(W), dev(s))
    q, z, sc = oracle.quantize_groups(oracle.scale_weights(W, s))
    codes, zeros = awq.awq_unpack(p, zd, K)
    assert np.array_equal(host(codes), q) and np.array_equal(host(zeros), z)
    x = activations_fp16(1, K, seed=43)
    y = host(awq.awq_gemm_scaled(dev(x), awq.awq_inverse_scale(dev(s)), p, scd, zd))
    ref = x.astype(np.float64) @ oracle.effective_weight(q, z, sc, s).T
    assert_y_close(y, ref, "end to end")
