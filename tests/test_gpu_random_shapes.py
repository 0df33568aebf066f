"""awq_gemm at seeded random shapes against the oracle, at both code widths: M from 1 to 300
and N from 1 to 3000 (every kernel of the dispatch and its partial tiles), K from 128 to
10240 in whole groups (odd group counts, fewer groups than waves).  Same bars as the other
product tests: relative Frobenius error <= 1e-3, max |dy| <= 1e-2 max |y_ref|."""
import numpy as np
import pytest

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16
from layout import assert_y_close
from test_gpu_parity import _random_packed, dev, host, note
from test_gpu_three_bit import _random_packed3

pytestmark = pytest.mark.gpu


def _shapes(seed, count):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        M = int(g.choice([int(g.integers(1, 17)), int(g.integers(17, 65)), int(g.integers(65, 301))]))
        N = int(g.integers(1, 3001))
        K = 128 * int(g.integers(1, 81))
        if N * K <= 4_000_000:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M,N,K", _shapes(2024, 24))
def test_gemm_random_shape(M, N, K, bits):
    note(f"random shape bits={bits} M={M} N={N} K={K}")
    seed = M * 7919 + N * 31 + K + bits
    q, z, sc, p, scd, zd = (_random_packed if bits == 4 else _random_packed3)(N, K, seed=seed)
    x = activations_fp16(M, K, seed=seed + 1)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=bits))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"bits={bits} M={M} N={N} K={K}")


def _search_shapes(seed, count):
    """(N, K, M): both loss forms (M < K direct, M >= K through the Gram matrix), row counts
    that leave partial 256-row tiles, K in whole groups that leave partial 256-channel blocks."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        N = int(g.integers(1, 401))
        K = 128 * int(g.integers(1, 9))
        M = int(g.choice([int(g.integers(1, K)), int(g.integers(K, 4 * K + 1))]))
        out.append((N, K, M))
    return out


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("N,K,M", _search_shapes(77, 6))
def test_search_random_shape(N, K, M, bits):
    """awq_quantize against the oracle's search: the alpha index up to ties within 1e-6
    relative loss, every loss within 1e-5 relative, and s, codes, zero points and steps at
    the chosen alpha bit-exact."""
    from gen import normal_fp16
    note(f"random search bits={bits} N={N} K={K} M={M}")
    seed = N * 131 + K * 7 + M + bits
    W = normal_fp16((N, K), 0.02, seed=seed)
    X = activations_fp16(M, K, seed=seed + 1, lognormal=bool(seed & 1))
    alphas = awq.default_alpha_grid(20)
    r = awq.awq_quantize(dev(W), dev(X), alphas, bits=bits)
    ref = oracle.search(W, X, alphas=alphas, bits=bits)
    best = int(host(r["best_alpha"])[0])
    L, Lg = ref["losses"], host(r["loss"])
    assert L[best] <= (1 + 1e-6) * L.min(), (best, ref["alpha_index"])
    nz = L > 0
    assert np.all(np.abs(Lg[nz] - L[nz]) <= 1e-5 * L[nz]), np.max(np.abs(Lg[nz] - L[nz]) / L[nz])
    assert np.all(Lg[~nz] == 0.0)
    q, z, sc, s = oracle.quantize_at(W, ref["a"], alphas[best], bits=bits)
    assert np.array_equal(host(r["s"]), s)
    codes, zz = awq.awq_unpack(r["packed"], r["zeros"], K)
    assert np.array_equal(host(codes), q) and np.array_equal(host(zz), z)
    assert np.array_equal(host(r["scales"]).view(np.uint16), sc.view(np.uint16))
