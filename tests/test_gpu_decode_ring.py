"""GPU parity of the matrix-core decode path (3 <= M <= 16) against the oracle, with the
bars of the other product tests (relative Frobenius error <= 1e-3, max |dy| <= 1e-2 max
|y_ref|), at shapes that select each ring layout: one or two 16-row tiles per wave, four
or eight waves per block.  Row counts leave a partial last block (which stages its scales
and zeros one by one instead of by DMA), group counts are odd or smaller than the wave
count, and one K is long enough that the block's scales and zeros no longer fit in LDS
beside the rings at M = 16, so the register-staged kernel runs instead."""
import numpy as np
import pytest

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16
from layout import assert_y_close
from test_gpu_parity import _random_packed, dev, host, note

pytestmark = pytest.mark.gpu


def _check(N, K, M, seed, sample=None):
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=seed)
    x = activations_fp16(M, K, seed=seed + 1)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    if sample is None:
        assert_y_close(y, oracle.gemm(x, q, z, sc), f"N={N} K={K} M={M}")
        return y
    g = np.random.default_rng(seed + 2)
    rows = np.union1d(g.choice(N, size=sample, replace=False), np.arange(N - 40, N))  # always the last block
    assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"N={N} K={K} M={M}")
    return y


@pytest.mark.parametrize("N,K,M", [
    (300, 384, 3), (300, 384, 6), (300, 384, 12), (300, 384, 16),  # 3 groups: 3 waves, ragged last block
    (47, 128, 5), (47, 128, 16),                                     # one group: one wave, one partial block
    (5, 256, 3), (5, 256, 16),                                       # fewer rows than one tile
    (300, 16640, 2), (64, 36096, 2),                                 # M = 2 on long rows
    (4090, 2176, 9),                                                 # one tile, eight waves; 17 groups
    (4100, 640, 7),                                                  # K <= 4096 on a wider layer: four waves
])
def test_ring_small_layers(N, K, M):
    note(f"ring N={N} K={K} M={M}")
    _check(N, K, M, seed=N * 3 + K + M)


@pytest.mark.parametrize("N,K,M", [
    (8190, 4224, 8), (8190, 4224, 13),  # two tiles, eight waves; 33 groups; 8190 = 255 * 32 + 30
    (9000, 4352, 6),                    # 8192 < N < 16384: one tile, four waves
    (16400, 4480, 9),                   # N >= 16384: two tiles, four waves; 16400 = 512 * 32 + 16
    (16400, 4480, 4),                   # M <= 4: one tile, eight waves
    (10240, 8192, 16), (12300, 8320, 9),  # K >= 8192, 8192 < N < 16384, M > 8: four tiles; 12300 = 192 * 64 + 12
    (16400, 8320, 13),                    # N >= 16384, K >= 8192, M > 8: four tiles, four waves
    (22016, 4096, 16),                    # N >= 16384, K < 8192, M > 8: two tiles, four waves
    (16400, 8320, 6), (22016, 4096, 7),   # the same for 4 < M <= 8
])
def test_ring_wide_layers_sampled_rows(N, K, M):
    note(f"ring N={N} K={K} M={M}")
    _check(N, K, M, seed=N + K * 5 + M, sample=256)


@pytest.mark.parametrize("M", [4, 16])
def test_ring_long_k(M):
    """K = 270336 (2112 groups): at M = 4 the block's scales and zeros (85 KB) still fit
    beside the rings; at M = 16 they do not, and the register-staged kernel runs."""
    note(f"ring long K M={M}")
    _check(64, 270336, M, seed=77 + M)


def test_ring_determinism():
    note("ring determinism")
    q, z, sc, p, scd, zd = _random_packed(8190, 4224, seed=12)
    for M in (3, 8, 16):
        x = dev(activations_fp16(M, 4224, seed=13 + M))
        a = host(awq.awq_gemm(x, p, scd, zd))
        b = host(awq.awq_gemm(x, p, scd, zd))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), M


@pytest.mark.parametrize("N,K,M", [(10240, 8192, 24), (12288, 6144, 32), (10240, 8192, 48), (12300, 4224, 17),
                                   (12288, 6144, 48), (16400, 8320, 24), (28672, 8192, 32)])
def test_ring_wide_layers_long_k(N, K, M):
    """17 <= M <= 64 on layers up to 12288 wide with K above 4096 (the 70B q/k/v shape) run
    on the ring with one weight tile per block up to M = 32 and two above; 12300 rows is just
    past that bound and takes the pipelined GEMM, as does K = 6144 above M = 32.  Wider layers
    with K >= 8192 (the 70B gate/up) take four tiles per block up to M = 32.  Checked on
    sampled rows and the last block."""
    note(f"multi-row N={N} K={K} M={M}")
    _check(N, K, M, seed=N + K + M, sample=256)


@pytest.mark.parametrize("N,K,M", [
    (4100, 4096, 20), (300, 640, 64),     # N <= 8192: one tile and two (M <= 32) or four x tiles; ragged blocks
    (1000, 16640, 24), (70, 28672, 32),   # K >= 16384, M <= 32: two tiles per block
    (11008, 4096, 32),                    # wider layer, K <= 4096, M <= 32
    (9000, 4096, 48),                     # wider layer above M = 32: the pipelined GEMM
    (100, 139264, 40),                    # K so long the block's scales leave the ring no LDS: fallback kernel
])
def test_ring_mid_m(N, K, M):
    """17 <= M <= 64 on the ring kernel with two or four 16-row x tiles per stage (each weight
    operand feeding that many MFMAs), on the layers where it is chosen; sampled rows on wide layers."""
    note(f"ring mid N={N} K={K} M={M}")
    _check(N, K, M, seed=N * 5 + K + M, sample=256 if N > 2000 else None)
