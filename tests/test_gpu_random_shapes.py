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
