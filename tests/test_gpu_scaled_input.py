"""GPU parity of the input side of the per-channel scaling against the oracle.

awq_scale_input must equal the oracle's x / s (one fp32 division, rounded once to fp16) bit for
bit.  awq_gemm_scaled must equal awq_gemm_bits on awq_scale_input's output bit for bit, and the
oracle's product on x / s to the usual bars (relative Frobenius error <= 1e-3, max |dy| <= 1e-2
max |y_ref|)."""
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


def _edge_input(M, K, seed):
    """Activations with signed zeros, fp16 subnormals, the largest fp16 values and ordinary
    values mixed, so that both signs of zero and both ends of the fp16 range are divided."""
    x = activations_fp16(M, K, seed=seed)
    g = np.random.default_rng(seed + 1)
    bits = x.view(np.uint16)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0x3C01, 0x7BFF, 0xFBFF],
                        dtype=np.uint16)
    idx = g.choice(M * K, size=min(M * K, 8 * len(specials)), replace=False)
    bits.reshape(-1)[idx] = specials[np.arange(idx.size) % len(specials)]
    return x


@pytest.mark.parametrize("M,K", [(1, 4096), (2, 11008), (37, 1024), (5, 8)])
def test_scale_input_bits(M, K):
    """awq_scale_input is the oracle's x / s, bit for bit (signed zeros included)."""
    note(f"scale input M={M} K={K}")
    s = _scales(K, 2 + K)
    s[:3] = [2.0 ** -45, 1.0, 65504.0]  # the ends of the range a search's s can take
    x = _edge_input(M, K, seed=3 + M)
    xs = host(awq.awq_scale_input(dev(x), dev(s)))
    ref = oracle.scaled_input(x, s)
    assert np.array_equal(xs.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("M,N,K,bits", [
    (1, 4096, 4096, 4), (2, 4096, 4096, 4), (1, 1000, 11008, 4), (2, 515, 2176, 4),  # decode GEMV
    (1, 11008, 4096, 4), (2, 4100, 4096, 4),
    (2, 300, 16384, 4),                                                                # M = 2, long rows
    (3, 700, 1024, 4), (16, 257, 2048, 4), (100, 300, 1024, 4),                        # matrix-core kernels
    (1, 600, 4096, 3), (7, 300, 1024, 3), (100, 300, 1024, 3),                         # 3-bit
])
def test_gemm_scaled_parity(M, N, K, bits):
    note(f"gemm scaled M={M} N={N} K={K} bits={bits}")
    seed = M + N + K + bits
    q, z, sc, p, scd, zd = (_random_packed if bits == 4 else _random_packed3)(N, K, seed=seed)
    s = _scales(K, seed + 1)
    x = activations_fp16(M, K, seed=seed + 2)
    y = host(awq.awq_gemm_scaled(dev(x), dev(s), p, scd, zd, bits=bits))
    xs = awq.awq_scale_input(dev(x), dev(s))
    assert np.array_equal(host(xs).view(np.uint16), oracle.scaled_input(x, s).view(np.uint16))
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
    y = host(awq.awq_gemm_scaled(dev(x), dev(s), p, scd, zd))
    ref = x.astype(np.float64) @ oracle.effective_weight(q, z, sc, s).T
    assert_y_close(y, ref, "end to end")
