"""The C++ oracle and the numpy implementation of the method agree.  The two are written
independently from the same readings (awq_oracle.cpp, awq_oracle.py); where the method is
integer or IEEE-exact (statistics, s, codes, zero points, steps, the chosen alpha, the scaled
input, the top-channel ranks) they must agree bit for bit, and where fp64 sums are formed in
different orders (losses, products) to 1e-12 relative."""
import numpy as np
import pytest

import oracle as C
from gen import activations_fp16, normal_fp16
from oracle import numpy_reference as P


@pytest.mark.parametrize("N,K,M,bits,gram", [(64, 512, 64, 4, False), (96, 640, 300, 3, True), (17, 128, 1, 4, False),
                                             (48, 256, 400, 4, True), (40, 384, 200, 4, False)])
def test_search_agrees(N, K, M, bits, gram):
    W = normal_fp16((N, K), 0.02, seed=N + K)
    X = activations_fp16(M, K, seed=M + K, lognormal=True)
    a, b = C.search(W, X, bits=bits, use_gram=gram), P.search(W, X, bits=bits, use_gram=gram)
    assert a["alpha_index"] == b["alpha_index"]
    assert np.array_equal(a["a"], b["a"]) and np.array_equal(a["s"], b["s"])
    for k in ("q", "z"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["scales"].view(np.uint16), b["scales"].view(np.uint16))
    assert np.allclose(a["losses"], b["losses"], rtol=1e-12, atol=0)


def test_quantizer_agrees_on_wide_values():
    g = np.random.default_rng(7)
    V = (g.standard_normal((64, 1024)) * np.exp2(g.integers(-20, 12, size=(64, 1)))).astype(np.float32)
    V[3, :128] = 0.0
    V[5, 128:256] = np.float32(3e-9)
    for bits in (3, 4):
        for x, y in zip(C.quantize_groups(V, bits=bits), P.quantize_groups(V, bits=bits)):
            assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


def test_products_and_scaled_input_agree():
    g = np.random.default_rng(8)
    N, K, M = 200, 1024, 7
    q = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = g.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    sc = (np.abs(g.standard_normal((N, K // 128))) * 0.01 + 1e-4).astype(np.float16)
    x = activations_fp16(M, K, seed=9)
    s = np.exp(g.normal(0, 1, K)).astype(np.float32)
    assert np.array_equal(C.scaled_input(x, s).view(np.uint16), P.scaled_input(x, s).view(np.uint16))
    assert np.allclose(C.gemm(x, q, z, sc), P.gemm(x, q, z, sc), rtol=1e-12, atol=1e-300)
    assert np.array_equal(C.dequantize(q, z, sc), P.dequantize(q, z, sc))
    assert np.array_equal(C.effective_weight(q, z, sc, s), P.effective_weight(q, z, sc, s))


def test_ablation_agrees():
    W = normal_fp16((64, 512), 0.02, seed=11)
    X = activations_fp16(600, 512, seed=12, lognormal=True)
    rnd = np.random.default_rng(13).permutation(512)[:5].astype(np.int32)
    for gram in (False, True):
        a, b = C.keep_fp16_ablation(W, X, 5, rnd, use_gram=gram), P.keep_fp16_ablation(W, X, 5, rnd, use_gram=gram)
        assert np.array_equal(a["keep_activation"], b["keep_activation"])
        assert np.array_equal(a["keep_weight"], b["keep_weight"])
        assert np.allclose(a["losses"], b["losses"], rtol=1e-12, atol=0)
