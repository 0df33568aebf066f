"""GPU parity: every libawq entry point against the CPU oracle on the same seeded inputs.

Bars: codes, zero points, steps, s, channel statistics and the chosen alpha index
bit-exact (the alpha index up to ties within 1e-6 relative loss); W4A16 outputs
within relative Frobenius error 1e-3 and max |dy| <= 1e-2 max |y_ref|; search losses
within 1e-5 relative of the oracle's (the device builds X^T X from fp32 partials of
256 calibration rows, the oracle in fp64).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16, normal_fp16, seed_for
from layout import assert_y_close, decode_codes, decode_zeros, encode
from test_oracle_pins import _on_grid_layer

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ALPHAS = awq.default_alpha_grid(20)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------------------ statistics
@pytest.mark.parametrize("M,K,seed,lognormal", [(64, 512, 1, False), (37, 384, 2, True), (1, 8, 3, False),
                                                (1000, 4096, 4, True), (513, 11008, 5, True)])
def test_channel_mean_abs_bit_exact(M, K, seed, lognormal):
    note(f"channel_mean_abs M={M} K={K}")
    X = activations_fp16(M, K, seed, lognormal=lognormal)
    a = host(awq.awq_channel_mean_abs(dev(X)))
    assert np.array_equal(a, oracle.channel_mean_abs(X))


def test_channel_mean_abs_extreme_values():
    note("channel_mean_abs extremes")
    g = np.random.default_rng(7)
    M, K = 700, 64  # spans three 256-row partial sums
    X = (g.choice([-1.0, 1.0], size=(M, K)) * g.choice([65504.0, 2.0 ** -24, 6.1e-5, 1.0, 0.0], size=(M, K)))
    X = X.astype(np.float16)
    a = host(awq.awq_channel_mean_abs(dev(X)))
    assert np.array_equal(a, oracle.channel_mean_abs(X))


# ------------------------------------------------------------------ packer
def _check_pack(W, s, packed, scales, zeros):
    N, K = W.shape
    q, z, sc = oracle.quantize_groups(oracle.scale_weights(W, np.ones(K, np.float32) if s is None else s))
    assert np.array_equal(decode_codes(host(packed), K), q)
    assert np.array_equal(decode_zeros(host(zeros), K // 128), z)
    assert np.array_equal(host(scales).view(np.uint16), sc.view(np.uint16))
    codes, zz = awq.awq_unpack(packed, zeros, K)
    assert np.array_equal(host(codes), q) and np.array_equal(host(zz), z)


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (100, 512), (7, 4096), (64, 11008)])
@pytest.mark.parametrize("scaled", [False, True])
def test_pack_bit_exact(N, K, scaled):
    note(f"pack N={N} K={K} scaled={scaled}")
    W = normal_fp16((N, K), 0.02, seed=100 + N + K)
    s = None
    if scaled:
        s = np.exp(np.random.default_rng(N * K).standard_normal(K) * 1.5).astype(np.float32)
    packed, scales, zeros = awq.awq_pack(dev(W), None if s is None else dev(s))
    _check_pack(W, s, packed, scales, zeros)


def test_pack_degenerate_groups():
    note("pack degenerate groups")
    K = 512
    W = normal_fp16((6, K), 0.02, seed=55)
    W[0] = 0                        # all-zero groups: floor step 2^-14
    W[1] = np.float16(0.125)        # constant positive
    W[2] = np.float16(-3.0)         # constant negative
    W[3, :128] = np.float16(60000)  # large magnitudes
    W[3, 128:256] = np.float16(-60000)
    W[4] = np.float16(6e-8)         # subnormal fp16 weights
    packed, scales, zeros = awq.awq_pack(dev(W))
    _check_pack(W, None, packed, scales, zeros)


# ------------------------------------------------------------------ search
def _check_search(W, X, r, ref, loss_rtol=1e-5):
    best = int(host(r["best_alpha"])[0])
    L = ref["losses"]
    Lg = host(r["loss"])
    assert L[best] <= (1 + 1e-6) * L.min(), f"alpha index {best} (L={L[best]}) vs oracle {ref['alpha_index']}"
    nz = L > 0
    assert np.all(np.abs(Lg[nz] - L[nz]) <= loss_rtol * L[nz]), np.max(np.abs(Lg[nz] - L[nz]) / L[nz])
    assert np.all(Lg[~nz] == 0.0)
    q, z, sc, s = oracle.quantize_at(W, ref["a"], ALPHAS[best])
    s_gpu = host(r["s"])
    assert np.array_equal(s_gpu, s), f"{np.sum(s_gpu != s)} of {s.size} s values differ"
    _check_pack(W, s, r["packed"], r["scales"], r["zeros"])
    return best


def test_search_single_layer_512():
    note("search single_layer_512")
    W = normal_fp16((512, 512), 0.02, seed=seed_for(1, 1))
    X = activations_fp16(64, 512, seed=seed_for(1, 2))
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    ref = oracle.search(W, X, alphas=ALPHAS)
    _check_search(W, X, r, ref)


@pytest.mark.parametrize("N,K,M,lognormal", [(100, 384, 50, False), (17, 128, 1, False), (96, 640, 300, True)])
def test_search_ragged(N, K, M, lognormal):
    note(f"search ragged N={N} K={K} M={M}")
    W = normal_fp16((N, K), 0.02, seed=N + K)
    X = activations_fp16(M, K, seed=M + 1, lognormal=lognormal)
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    _check_search(W, X, r, oracle.search(W, X, alphas=ALPHAS))


def test_search_forced_tie():
    note("search forced tie")
    g = np.random.default_rng(50)
    X = (g.choice([-4.0, 4.0], size=(32, 256))).astype(np.float16)
    W = normal_fp16((16, 256), 0.02, seed=51)
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    ref = oracle.search(W, X, alphas=ALPHAS)
    best = _check_search(W, X, r, ref)
    Lg = host(r["loss"])
    assert Lg[10] == Lg[0] and best != 10


def test_search_known_answer():
    note("search known answer")
    W, X, c, z0 = _on_grid_layer()
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    assert int(host(r["best_alpha"])[0]) == 10
    Lg = host(r["loss"])
    assert Lg[10] == 0.0 and np.all(np.delete(Lg, 10) > 0)
    codes, zz = awq.awq_unpack(r["packed"], r["zeros"], W.shape[1])
    assert np.array_equal(host(codes), c) and np.array_equal(host(zz), z0)


@pytest.mark.parametrize("N,K,M", [(512, 4096, 4096), (256, 11008, 2048)])
def test_search_llama_shaped(N, K, M):
    note(f"search llama-shaped N={N} K={K} M={M}")
    W = normal_fp16((N, K), 0.02, seed=5000 + K)
    X = activations_fp16(M, K, seed=5001 + K, lognormal=True)
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    ref = oracle.search(W, X, alphas=ALPHAS)
    best = _check_search(W, X, r, ref)
    note(f"  alpha*={ALPHAS[best]:.2f} L(alpha*)/L(0)={ref['losses'][best] / ref['losses'][0]:.4f}")


@pytest.mark.parametrize("widths,K,M", [((192, 128, 128), 512, 1024), ((256, 256), 384, 200)])
def test_search_joint_shared_input(widths, K, M):
    """Layers reading the same input (q/k/v, gate/up) searched jointly for one s: awq_quantize on
    their row-concatenated weights.  Its loss at every alpha is the row-weighted mean of the
    layers' own output MSEs (checked against the oracle per layer), so alpha* minimizes their sum;
    the packed result is the fused matrix the decode path multiplies, and it is checked against
    the oracle's search on the concatenation like any other layer."""
    note(f"joint search widths={widths} K={K} M={M}")
    Ws = [normal_fp16((n, K), 0.02, seed=600 + i) for i, n in enumerate(widths)]
    X = activations_fp16(M, K, seed=601, lognormal=True)
    Wc = np.concatenate(Ws, axis=0)
    r = awq.awq_quantize(dev(Wc), dev(X), ALPHAS)
    ref = oracle.search(Wc, X, alphas=ALPHAS)
    _check_search(Wc, X, r, ref)
    parts = [oracle.search(W, X, alphas=ALPHAS)["losses"] for W in Ws]
    mean = sum(n * L for n, L in zip(widths, parts)) / sum(widths)
    assert np.allclose(ref["losses"], mean, rtol=1e-12, atol=0)
    assert np.allclose(host(r["loss"]), mean, rtol=1e-5, atol=0)


def test_search_determinism():
    note("search determinism")
    W = normal_fp16((256, 512), 0.02, seed=77)
    X = activations_fp16(300, 512, seed=78)
    r1 = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    r2 = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    for k in ("packed", "scales", "zeros", "s", "best_alpha", "loss"):
        assert np.array_equal(host(r1[k]).view(np.uint8), host(r2[k]).view(np.uint8)), k


@pytest.mark.parametrize("K,M", [(512, 700), (512, 300)])  # Gram form (M >= K), direct form (M < K)
def test_search_reused_statistics(K, M):
    """Layers on one input searched one after another on one workspace, the later ones taking
    the statistics of X from it (awq_quantize_shared): every output equals a search that
    recomputes them, bit for bit, whatever N, bits and alpha grid the earlier layer had; the
    first layer is checked against the oracle."""
    note(f"search reused statistics K={K} M={M}")
    X = dev(activations_fp16(M, K, seed=88, lognormal=True))
    layers = [(384, 4, ALPHAS), (128, 4, ALPHAS[:7]), (256, 3, ALPHAS)]
    Ws = [dev(normal_fp16((n, K), 0.02, seed=89 + i)) for i, (n, _, _) in enumerate(layers)]
    need = max(awq.awq_quantize_workspace_bytes(n, K, M, 128, len(al)) for n, _, al in layers)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    for i, ((n, bits, al), W) in enumerate(zip(layers, Ws)):
        shared = awq.awq_quantize(W, X, al, workspace=ws, bits=bits, reuse_statistics=i > 0)
        fresh = awq.awq_quantize(W, X, al, bits=bits)
        for k in ("packed", "scales", "zeros", "s", "best_alpha", "loss"):
            assert np.array_equal(host(shared[k]).view(np.uint8), host(fresh[k]).view(np.uint8)), (i, k)
        if i == 0:
            Wh = host(W)
            _check_search(Wh, host(X), shared, oracle.search(Wh, host(X), alphas=al, bits=bits))


# ------------------------------------------------------------------ W4A16 product
def _random_packed(N, K, seed, sigma=0.02):
    g = np.random.default_rng(seed)
    q = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = g.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    sc = (np.abs(g.standard_normal((N, K // 128))) * sigma * 0.4 + 1e-4).astype(np.float16)
    p, zb = encode(q, z)
    return q, z, sc, dev(p), dev(sc), dev(zb)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 33, 64, 100, 256])
def test_gemm_parity_ragged(M):
    note(f"gemm M={M} N=300 K=1024")
    N, K = 300, 1024
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=M)
    x = activations_fp16(M, K, seed=900 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"M={M}")


@pytest.mark.parametrize("N,K,M", [(77, 384, 17), (77, 384, 64), (77, 384, 65), (77, 384, 130), (131, 640, 200),
                                   (200, 16640, 70), (136, 16640, 40), (72, 33280, 70), (72, 36096, 70),
                                   (64, 36096, 20), (8200, 512, 17), (8200, 512, 40), (8200, 512, 50),
                                   (28672, 512, 128)])
def test_gemm_parity_block_tails(N, K, M):
    """Weight-row counts that leave a partial 128-row block, odd group counts (the block's
    scales and zeros end off a 16-byte boundary), K = 16640 (130 groups: 64-row tiles over
    four stages), K = 33280 (260 groups: 64-row tiles over three stages, one channel set),
    K = 36096 (282 groups, more than any pipelined layout holds, so the general-shape kernel
    runs), 28672 rows at M = 128 (128-row tiles, which fill the chip there); N = 8200 with
    17 <= M <= 32 takes the multi-m-tile decode kernel with four tiles per wave, larger M
    the GEMM's 64-row tiles."""
    note(f"gemm tails N={N} K={K} M={M}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=N + K + M)
    x = activations_fp16(M, K, seed=40 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"N={N} K={K} M={M}")


@pytest.mark.parametrize("K", [2048, 4096, 8192, 16384, 32768, 6144, 12288])
@pytest.mark.parametrize("N", [512, 520])
@pytest.mark.parametrize("M", [8, 100])
def test_gemm_parity_scale_layouts(K, N, M):
    """The matrix-core kernels stage a block's group scales in LDS with a row-dependent
    permutation of 16-byte pieces where a row of scales is a power-of-two number of pieces
    (G = K / 128 = 16 .. 256 here); G = 48 and 96 keep the plain layout.  M = 8 runs the decode
    ring kernel, M = 100 the pipelined GEMM; N = 520 leaves a ragged last block, whose scales
    are copied element by element into the same layout.  Every (row, group) scale is distinct,
    so a misplaced one shows in y."""
    note(f"gemm scale layout K={K} N={N} M={M}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=K + N + M)
    x = activations_fp16(M, K, seed=77 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"K={K} N={N} M={M}")


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_gemm_one_hot_reproduces_dequantized_column(M):
    note(f"gemm one-hot M={M}")
    N, K = 80, 512
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=31 + M)
    ks = [0, 1, 7, 8, 127, 128, 300, 511, 2, 129, 255, 256, 383, 384, 400, 510][:M]
    x = np.zeros((M, K), np.float16)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    for m, k in enumerate(ks):
        col = (q[:, k].astype(np.float64) - z[:, k // 128]) * sc[:, k // 128].astype(np.float64)
        assert np.array_equal(y[m], col.astype(np.float16)), (m, k)


@pytest.mark.parametrize("M,N", [(1, 80), (2, 80), (3, 80), (5, 80), (9, 80), (16, 80), (24, 80), (40, 80),
                                 (64, 80), (100, 80), (256, 80), (512, 8192)])
def test_gemm_one_hot_every_code_position_exact(M, N):
    """Row m of x is the unit vector of channel 37 m mod K (37 is odd, so the channels cover all
    eight nibble positions of a packed word, all four words of a 16-byte piece and all four
    groups), with unit scales and every (code, zero) pair present: y[m][n] must equal
    code - zero exactly, on whichever kernel the M class takes (GEMV, decode ring, matrix-core
    ring and pipelined GEMM with 64- and 128-row tiles)."""
    K = 512
    kernel = awq.awq_gemm_kernel(M, N, K)
    note(f"gemm one-hot every position M={M}: {kernel}")
    n = np.arange(N)[:, None]
    q = ((n + np.arange(K)[None, :] * 5) % 16).astype(np.uint8)        # every code on every row
    z = ((n * 3 + np.arange(K // 128)[None, :] * 7) % 16).astype(np.uint8)  # every zero point
    sc = np.ones((N, K // 128), np.float16)
    p, zb = encode(q, z)
    pd, scd, zbd = dev(p), dev(sc), dev(zb)
    for shift in range(16 if M <= 2 else 1):  # one or two channels per launch: 16 launches
        ks = [(37 * (m + M * shift)) % K for m in range(M)]
        x = np.zeros((M, K), np.float16)
        x[np.arange(M), ks] = 1.0
        y = host(awq.awq_gemm(dev(x), pd, scd, zbd))
        want = (q[:, ks].astype(np.int32) - z[:, np.array(ks) // 128].astype(np.int32)).T.astype(np.float16)
        assert np.array_equal(y.view(np.uint16), want.view(np.uint16)), \
            f"M={M} ({kernel}) shift {shift}: first mismatch at {np.argwhere(y != want)[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (2, 64, 256), (5, 64, 256), (8, 64, 256), (9, 64, 256),
                                   (64, 64, 256), (1, 4096, 4096), (2, 11008, 4096), (1, 4096, 11008),
                                   (1, 8192, 28672), (16, 300, 4096), (256, 300, 4096)])
def test_gemm_codes_equal_zeros_gives_zero(M, N, K):
    """Every code equal to its zero point: w_hat = 0, so y = 0 exactly on every kernel (each
    subtracts the zero point per code before any product)."""
    note(f"gemm zero codes M={M} N={N} K={K}")
    g = np.random.default_rng(5)
    z = g.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    q = np.repeat(z, 128, axis=1)
    sc = np.full((N, K // 128), 0.01, np.float16)
    p, zb = encode(q, z)
    x = activations_fp16(M, K, seed=6)
    y = host(awq.awq_gemm(dev(x), dev(p), dev(sc), dev(zb))).astype(np.float64)
    assert np.all(y == 0), f"M={M} N={N} K={K}: max |y| {np.abs(y).max()}"


def test_gemm_quantized_layer_end_to_end():
    """x / s through the packed layer the search produced equals the oracle's product."""
    note("gemm after search")
    W = normal_fp16((512, 512), 0.02, seed=seed_for(1, 1))
    X = activations_fp16(64, 512, seed=seed_for(1, 2))
    r = awq.awq_quantize(dev(W), dev(X), ALPHAS)
    best = int(host(r["best_alpha"])[0])
    q, z, sc, s = oracle.quantize_at(W, oracle.channel_mean_abs(X), ALPHAS[best])
    for M in (1, 4):
        x = (activations_fp16(M, 512, seed=seed_for(1, 3 + M)).astype(np.float32) / s).astype(np.float16)
        y = host(awq.awq_gemm(dev(x), r["packed"], r["scales"], r["zeros"]))
        assert_y_close(y, oracle.gemm(x, q, z, sc), f"M={M}")


_7B = [(4096, 4096), (4096, 11008), (11008, 4096)]
_70B = [(8192, 10240), (8192, 8192), (8192, 28672), (28672, 8192)]


@pytest.mark.parametrize("K,N", _7B)
def test_gemv_llama2_7b_decode_full(K, N):
    note(f"7B decode GEMV K={K} N={N}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=K + N)
    x = activations_fp16(1, K, seed=K)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"K={K} N={N}")


@pytest.mark.parametrize("K,N", _70B)
@pytest.mark.parametrize("M", [1, 8, 16])
def test_gemm_llama2_70b_sampled_rows(K, N, M):
    note(f"70B K={K} N={N} M={M}")
    g = np.random.default_rng(K * 3 + N)
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=K * 7 + N, sigma=0.015)
    x = activations_fp16(M, K, seed=K + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    rows = np.sort(g.choice(N, size=384, replace=False))
    assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"K={K} N={N} M={M}")


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_batch_sweep_4096x11008(M):
    note(f"batch sweep M={M}")
    K, N = 4096, 11008
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=3)
    x = activations_fp16(M, K, seed=3000 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"M={M}")


@pytest.mark.parametrize("M", [1, 2, 8, 64])
def test_gemm_fused_rows_equal_separate_layers(M):
    """q/k/v (or gate/up) stored as one packed matrix with their rows concatenated give, bit for
    bit, the outputs of the separate layers side by side: every output row is computed from its
    own weight row alone, whatever the kernel's row blocking."""
    note(f"fused rows M={M}")
    K = 1024
    parts = [_random_packed(N, K, seed=70 + N) for N in (384, 256, 320)]
    x = dev(activations_fp16(M, K, seed=71 + M))
    ys = [host(awq.awq_gemm(x, p, scd, zd)) for (_, _, _, p, scd, zd) in parts]
    cat = [torch.cat([part[i] for part in parts], dim=0) for i in (3, 4, 5)]
    yf = host(awq.awq_gemm(x, *cat))
    assert np.array_equal(yf.view(np.uint16), np.concatenate(ys, axis=1).view(np.uint16))


@pytest.mark.parametrize("M", [1 << 22, (1 << 22) - 3])
def test_gemm_largest_m(M):
    """The largest M the boundary accepts (2^22 rows) with K = 1024: x holds 2^32 elements, so
    any 32-bit offset into x or y would wrap.  x is drawn on the device from a seeded generator
    (8 GB); sampled rows, among them those on both sides of element 2^31 and the last ones
    (the ragged last tile when M = 2^22 - 3), are checked against the oracle."""
    N, K = 48, 1024
    note(f"gemm largest M={M} N={N} K={K}: {awq.awq_gemm_kernel(M, N, K)}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=77)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(78)
    x = torch.randn((M, K), generator=gen, device="cuda:0", dtype=torch.float16)
    y = awq.awq_gemm(x, p, scd, zd)
    rng = np.random.default_rng(79)
    edge = (1 << 31) // K  # first row whose elements lie at or past 2^31
    rows = np.unique(np.concatenate([[0, 1, 2, edge - 2, edge - 1, edge, edge + 1, M - 3, M - 2, M - 1],
                                     rng.integers(0, M, size=22)]))
    idx = torch.from_numpy(rows).to("cuda:0")
    xs = host(x.index_select(0, idx))
    ys = host(y.index_select(0, idx))
    del x, y
    torch.cuda.empty_cache()
    assert_y_close(ys, oracle.gemm(xs, q, z, sc), f"largest M={M}")


@pytest.mark.parametrize("M", [1, 16, 24, 100])
def test_gemm_largest_k(M):
    """The largest K the boundary accepts (2^20 channels, 8192 groups per row): the register-staged
    and general-shape kernels that take layers whose scales and zeros leave the LDS rings no room."""
    N, K = 40, 1 << 20
    note(f"gemm largest K M={M} N={N} K={K}: {awq.awq_gemm_kernel(M, N, K)}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=80 + M)
    x = activations_fp16(M, K, seed=81 + M)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    assert_y_close(y, oracle.gemm(x, q, z, sc), f"largest K M={M}")


def test_gemm_determinism():
    note("gemm determinism")
    q, z, sc, p, scd, zd = _random_packed(1000, 2048, seed=8)
    for M in (1, 8, 100):
        x = dev(activations_fp16(M, 2048, seed=9))
        a = host(awq.awq_gemm(x, p, scd, zd))
        b = host(awq.awq_gemm(x, p, scd, zd))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


# ------------------------------------------------------------------ full-size search (stored oracle results)
def test_search_llama2_7b_block_full():
    """The 7B-block search workload at full size (65,536 calibration rows per input, seven
    layers) against the oracle's results stored by tests/golden/make_search_llama2_7b_block.py:
    alpha index within the tie rule, losses within 1e-5, and the packed layer at alpha*
    bit-exact against the oracle's quantizer (recomputed here; it needs no loss)."""
    import json
    import os
    from gen.workloads import layer_inputs_7b_block
    golden = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "search_llama2_7b_block.json")))
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_search_llama2_7b_block as mk
    alphas = np.array(golden["alphas"], dtype=np.float32)
    assert np.array_equal(alphas, ALPHAS)
    cache = {}
    for li, (lname, src) in enumerate(layer_inputs_7b_block()):
        ref = golden["layers"][lname]
        K, N = ref["K"], ref["N"]
        note(f"7B block search {lname} K={K} N={N} M={golden['calib_rows']}")
        if src not in cache:
            cache.clear()
            Xh = mk.calib_input(src)
            cache[src] = (Xh, dev(Xh), oracle.channel_mean_abs(Xh))
        Xh, Xd, a = cache[src]
        W = mk.layer_weight(li, K, N)
        r = awq.awq_quantize(dev(W), Xd, ALPHAS)
        best = int(host(r["best_alpha"])[0])
        L = np.array(ref["losses"])
        Lg = host(r["loss"])
        assert L[best] <= (1 + 1e-6) * L.min(), (lname, best, ref["alpha_index"])
        assert np.all(np.abs(Lg - L) <= 1e-5 * L), (lname, np.max(np.abs(Lg - L) / L))
        q, z, sc, s = oracle.quantize_at(W, a, ALPHAS[best])
        assert np.array_equal(host(r["s"]), s), lname
        assert np.array_equal(decode_codes(host(r["packed"]), K), q), lname
        assert np.array_equal(decode_zeros(host(r["zeros"]), K // 128), z), lname
        assert np.array_equal(host(r["scales"]).view(np.uint16), sc.view(np.uint16)), lname
        del r
        torch.cuda.empty_cache()
