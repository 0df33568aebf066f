"""GPU parity of the 3-bit format against the oracle at bits=3, with the bars of the 4-bit
path: codes, zero points, steps, s and the alpha index bit-exact (the index up to ties
within 1e-6 relative loss); products within relative Frobenius error 1e-3 and
max |dy| <= 1e-2 max |y_ref|."""
import numpy as np
import pytest

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16, normal_fp16
from layout import assert_y_close, decode_codes3, decode_zeros, encode3
from test_gpu_parity import ALPHAS, dev, host, note

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ packer
def _check_pack3(W, s, packed, scales, zeros):
    N, K = W.shape
    q, z, sc = oracle.quantize_groups(oracle.scale_weights(W, np.ones(K, np.float32) if s is None else s), bits=3)
    assert tuple(packed.shape) == (N, 3 * K // 32)
    assert np.array_equal(decode_codes3(host(packed), K), q)
    assert np.array_equal(decode_zeros(host(zeros), K // 128), z)
    assert np.array_equal(host(scales).view(np.uint16), sc.view(np.uint16))
    codes, zz = awq.awq_unpack(packed, zeros, K)  # the width follows from the packed shape
    assert np.array_equal(host(codes), q) and np.array_equal(host(zz), z)


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (100, 512), (7, 4096), (64, 11008)])
@pytest.mark.parametrize("scaled", [False, True])
def test_pack3_bit_exact(N, K, scaled):
    note(f"pack3 N={N} K={K} scaled={scaled}")
    W = normal_fp16((N, K), 0.02, seed=300 + N + K)
    s = None
    if scaled:
        s = np.exp(np.random.default_rng(N + K).standard_normal(K) * 1.5).astype(np.float32)
    packed, scales, zeros = awq.awq_pack(dev(W), None if s is None else dev(s), bits=3)
    _check_pack3(W, s, packed, scales, zeros)


def test_pack3_degenerate_groups():
    note("pack3 degenerate groups")
    K = 512
    W = normal_fp16((6, K), 0.02, seed=56)
    W[0] = 0
    W[1] = np.float16(0.125)
    W[2] = np.float16(-3.0)
    W[3, :128] = np.float16(60000)
    W[3, 128:256] = np.float16(-60000)
    W[4] = np.float16(6e-8)
    packed, scales, zeros = awq.awq_pack(dev(W), bits=3)
    _check_pack3(W, None, packed, scales, zeros)


# ------------------------------------------------------------------ search
@pytest.mark.parametrize("N,K,M,lognormal", [(512, 512, 64, False), (100, 384, 50, False), (96, 640, 300, True),
                                             (256, 1024, 2048, True)])
def test_search3(N, K, M, lognormal):
    """Direct (M < K) and Gram (M >= K) forms of the loss at 3 bits."""
    note(f"search3 N={N} K={K} M={M}")
    W = normal_fp16((N, K), 0.02, seed=700 + N + K)
    X = activations_fp16(M, K, seed=701 + M, lognormal=lognormal)
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS, bits=3)
    ref = oracle.search(W, X, alphas=ALPHAS, bits=3)
    best = int(host(r["best_alpha"])[0])
    L = ref["losses"]
    Lg = host(r["loss"])
    assert L[best] <= (1 + 1e-6) * L.min(), f"alpha index {best} vs oracle {ref['alpha_index']}"
    assert np.all(np.abs(Lg - L) <= 1e-5 * L)
    q, z, sc, s = oracle.quantize_at(W, ref["a"], ALPHAS[best], bits=3)
    assert np.array_equal(host(r["s"]), s)
    _check_pack3(W, s, r["packed"], r["scales"], r["zeros"])
    # 3-bit codes lose more than 4-bit ones on the same layer
    assert L.min() > oracle.search(W, X, alphas=ALPHAS, bits=4)["losses"].min()


# ------------------------------------------------------------------ product
def _random_packed3(N, K, seed, sigma=0.02):
    g = np.random.default_rng(seed)
    q = g.integers(0, 8, size=(N, K)).astype(np.uint8)
    z = g.integers(0, 8, size=(N, K // 128)).astype(np.uint8)
    sc = (np.abs(g.standard_normal((N, K // 128))) * sigma * 0.8 + 1e-4).astype(np.float16)
    p, zb = encode3(q, z)
    return q, z, sc, dev(p), dev(sc), dev(zb)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16, 33, 64, 100, 256])
def test_gemm3_parity_ragged(M):
    note(f"gemm3 M={M} N=300 K=1024")
    q, z, sc, p, scd, zd = _random_packed3(300, 1024, seed=M)
    x = activations_fp16(M, 1024, seed=950 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"M={M}")


@pytest.mark.parametrize("N,K,M", [(77, 384, 1), (77, 384, 2), (77, 384, 17), (131, 640, 200), (200, 16640, 1),
                                   (200, 16640, 70), (64, 36096, 2), (8200, 512, 40), (4096, 4096, 1),
                                   (4096, 11008, 1), (11008, 4096, 2), (8192, 8192, 1)])
def test_gemm3_parity_shapes(N, K, M):
    """Partial row blocks, 130 groups, K beyond the GEMV's 32768 (the matrix-core kernel then
    serves M = 2), and the 7B/70B decode shapes in full."""
    note(f"gemm3 N={N} K={K} M={M}")
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=N + K + M)
    x = activations_fp16(M, K, seed=60 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=3))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"N={N} K={K} M={M}")


@pytest.mark.parametrize("M", [1, 100])
def test_gemm3_largest_k(M):
    """3 bits at the largest K the boundary accepts (2^20 channels): the general-shape kernel."""
    N, K = 40, 1 << 20
    note(f"gemm3 largest K M={M} N={N} K={K}: {awq.awq_gemm_kernel(M, N, K, bits=3)}")
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=90 + M)
    x = activations_fp16(M, K, seed=91 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=3))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"3-bit largest K M={M}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm3_one_hot_reproduces_dequantized_column(M):
    note(f"gemm3 one-hot M={M}")
    N, K = 80, 512
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=41 + M)
    ks = [0, 1, 30, 31, 127, 128, 300, 511, 2, 29, 62, 63, 383, 384, 400, 510][:M]
    x = np.zeros((M, K), np.float16)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    for m, k in enumerate(ks):
        col = (q[:, k].astype(np.float64) - z[:, k // 128]) * sc[:, k // 128].astype(np.float64)
        assert np.array_equal(y[m], col.astype(np.float16)), (m, k)


@pytest.mark.parametrize("M,N", [(1, 80), (2, 80), (5, 80), (16, 80), (24, 80), (64, 80), (256, 80), (512, 8192)])
def test_gemm3_one_hot_every_code_position_exact(M, N):
    """3-bit twin of the 4-bit exact one-hot test: row m of x is the unit vector of channel
    37 m mod K (all 32 positions of a three-word chunk, the two spare-bit channels included),
    unit scales, every (code, zero) pair present; y[m][n] = code - zero exactly."""
    K = 512
    kernel = awq.awq_gemm_kernel(M, N, K, bits=3)
    note(f"gemm3 one-hot every position M={M}: {kernel}")
    n = np.arange(N)[:, None]
    q = ((n + np.arange(K)[None, :] * 3) % 8).astype(np.uint8)
    z = ((n * 5 + np.arange(K // 128)[None, :] * 3) % 8).astype(np.uint8)
    sc = np.ones((N, K // 128), np.float16)
    p, zb = encode3(q, z)
    pd, scd, zbd = dev(p), dev(sc), dev(zb)
    for shift in range(16 if M <= 2 else 1):  # one or two channels per launch: 16 launches
        ks = [(37 * (m + M * shift)) % K for m in range(M)]
        x = np.zeros((M, K), np.float16)
        x[np.arange(M), ks] = 1.0
        y = host(awq.awq_gemm(dev(x), pd, scd, zbd, bits=3))
        want = (q[:, ks].astype(np.int32) - z[:, np.array(ks) // 128].astype(np.int32)).T.astype(np.float16)
        assert np.array_equal(y.view(np.uint16), want.view(np.uint16)), \
            f"M={M} ({kernel}) shift {shift}: first mismatch at {np.argwhere(y != want)[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (2, 64, 256), (5, 64, 256), (64, 64, 256), (1, 4096, 4096),
                                   (2, 1000, 11008), (16, 300, 4096), (100, 300, 1024)])
def test_gemm3_codes_equal_zeros_gives_zero(M, N, K):
    """Every code equal to its zero point: w_hat = 0, so y = 0 exactly on every kernel (each
    subtracts the zero point per code before any product)."""
    note(f"gemm3 zero codes M={M} N={N} K={K}")
    z = np.random.default_rng(6).integers(0, 8, size=(N, K // 128)).astype(np.uint8)
    q = np.repeat(z, 128, axis=1)
    sc = np.full((N, K // 128), 0.01, np.float16)
    p, zb = encode3(q, z)
    x = activations_fp16(M, K, seed=7)
    y = host(awq.awq_gemm(dev(x), dev(p), dev(sc), dev(zb))).astype(np.float64)
    assert np.all(y == 0), f"M={M} N={N} K={K}: max |y| {np.abs(y).max()}"


def test_gemm3_after_search_end_to_end():
    """x / s through the 3-bit layer the search produced equals the oracle's product."""
    note("gemm3 after search")
    W = normal_fp16((512, 512), 0.02, seed=901)
    X = activations_fp16(64, 512, seed=902)
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS, bits=3)
    best = int(host(r["best_alpha"])[0])
    q, z, sc, s = oracle.quantize_at(W, oracle.channel_mean_abs(X), ALPHAS[best], bits=3)
    for M in (1, 4, 100):
        x = (activations_fp16(M, 512, seed=903 + M).astype(np.float32) / s).astype(np.float16)
        y = host(awq.awq_gemm(dev(x), r["packed"], r["scales"], r["zeros"]))
        assert_y_close(y, oracle.gemm(x, q, z, sc), f"M={M}")


@pytest.mark.parametrize("N,K,M", [(300, 384, 3), (300, 384, 16), (47, 128, 5), (5, 256, 12), (4090, 2176, 9), (4100, 640, 7),
                                   (64, 270336, 4), (64, 270336, 16)])
def test_gemm3_decode_ring(N, K, M):
    """3 <= M <= 16 on the LDS-ring decode kernel with 48-byte rows: 1, 3 and 17 groups
    (fewer chunks than waves), ragged last blocks, one- and four-wave layouts, and a long K
    where the block's scales no longer fit beside the rings at M = 16 (the general
    matrix-core kernel then runs)."""
    note(f"gemm3 ring N={N} K={K} M={M}")
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=N * 5 + K + M)
    x = activations_fp16(M, K, seed=70 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=3))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"N={N} K={K} M={M}")


@pytest.mark.parametrize("N,K,M", [(8190, 4224, 8), (9000, 4352, 6), (16400, 4480, 9), (16400, 4480, 4),
                                   (10240, 8192, 16), (12300, 8320, 11),   # four 16-row tiles per block
                                   (16400, 8320, 12)])
def test_gemm3_decode_ring_wide_sampled_rows(N, K, M):
    """Two tiles per wave with eight or four waves, and one tile with four, on wide layers
    with a partial last block (sampled rows, always including the last block's)."""
    note(f"gemm3 ring N={N} K={K} M={M}")
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=N + 3 * K + M)
    x = activations_fp16(M, K, seed=71 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=3))
    g = np.random.default_rng(N + M)
    rows = np.union1d(g.choice(N, size=256, replace=False), np.arange(N - 40, N))
    assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"N={N} K={K} M={M}")


@pytest.mark.parametrize("N,K,M", [(300, 640, 40), (1000, 16640, 24), (4100, 4096, 64), (11008, 4096, 20),
                                   (10240, 8192, 24), (10240, 8192, 48), (9000, 4224, 50), (16400, 8320, 24),
                                   (16400, 6144, 24), (10240, 6144, 48)])
def test_gemm3_ring_mid_m(N, K, M):
    """17 <= M <= 64 at 3 bits on the ring kernel with two or four x tiles per stage.  Most of
    these shapes have a ring layout of their own (the 4-bit rule); layers with none at 3 bits
    take the fallback layout: (16400, 6144) at M = 24 (wider than 12288 rows with
    4096 < K < 8192: one weight tile per block) and (10240, 6144) and (9000, 4224) above M = 32
    (two weight tiles per block)."""
    note(f"gemm3 ring mid N={N} K={K} M={M}")
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=N + K + M)
    x = activations_fp16(M, K, seed=N + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=3))
    if N > 2000:
        rows = np.union1d(np.random.default_rng(M).choice(N, size=256, replace=False), np.arange(N - 40, N))
        assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"N={N} K={K} M={M}")
    else:
        assert_y_close(y, oracle.gemm(x, q, z, sc), f"N={N} K={K} M={M}")


@pytest.mark.parametrize("N,K,M", [(11008, 4096, 256), (4096, 11008, 100), (1000, 4224, 130), (300, 1024, 1000),
                                   (64, 139264, 70), (11008, 4096, 64), (28672, 8192, 48), (12300, 4224, 50)])
def test_gemm3_pipelined_large_m(N, K, M):
    """M > 64 at 3 bits on the pipelined matrix-core GEMM (64- and 128-row tiles, ragged row and
    column blocks, 33 groups), and 32 < M <= 64 on the widest layers or short K, where the
    ring has no layout of its own; on K = 139264 the block's scales no longer fit beside the pipeline and the
    general-shape kernel runs.  Sampled rows on wide layers."""
    note(f"gemm3 pipe N={N} K={K} M={M}")
    q, z, sc, p, scd, zd = _random_packed3(N, K, seed=N + K + M)
    x = activations_fp16(M, K, seed=N + 2 * M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd, bits=3))
    if N > 2000:
        rows = np.union1d(np.random.default_rng(M).choice(N, size=256, replace=False), np.arange(N - 40, N))
        assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"N={N} K={K} M={M}")
    else:
        assert_y_close(y, oracle.gemm(x, q, z, sc), f"N={N} K={K} M={M}")
