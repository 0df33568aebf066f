"""Every kernel the product dispatch can launch (tests/dispatch_shapes.py), run once on the
GPU against the oracle with the product bars (relative Frobenius error <= 1e-3, max |dy| <=
1e-2 max |y_ref|); wide layers on sampled rows plus the last block."""
import numpy as np
import pytest

import oracle
import weight_only_quantization_gemm_amd as awq
from dispatch_shapes import BRANCHES, STREAMK_BRANCHES
from gen import activations_fp16
from layout import assert_y_close
from test_gpu_parity import _random_packed, dev, host, note
from test_gpu_three_bit import _random_packed3

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,shape", BRANCHES, ids=[n for n, _ in BRANCHES])
def test_each_dispatched_kernel(name, shape):
    M, N, K, bits = shape
    note(f"dispatch {name} M={M} N={N} K={K} bits={bits}")
    assert awq.awq_gemm_kernel(M, N, K, bits=bits, workspace=False).split(" ")[0] == name
    _run(name, M, N, K, bits, workspace=None)


@pytest.mark.parametrize("name,shape", STREAMK_BRANCHES, ids=[n + "-stream-K" for n, _ in STREAMK_BRANCHES])
def test_each_streamk_kernel(name, shape):
    M, N, K, bits = shape
    note(f"dispatch stream-K {name} M={M} N={N} K={K} bits={bits}")
    assert awq.awq_gemm_kernel(M, N, K, bits=bits).endswith("stream-K")
    _run(name, M, N, K, bits, workspace="auto")


def _run(name, M, N, K, bits, workspace):
    seed = M * 7 + N * 3 + K + bits
    q, z, sc, p, scd, zd = (_random_packed3 if bits == 3 else _random_packed)(N, K, seed=seed)
    x = activations_fp16(M, K, seed=seed + 1)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, workspace=workspace))
    if N <= 300:
        rows = np.arange(N)
    else:
        g = np.random.default_rng(seed + 2)
        rows = np.union1d(g.choice(N, size=128, replace=False), np.arange(N - 40, N))
    assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"{name} M={M} N={N} K={K}")
