"""The GEMM's stream-K split (awq_gemm_ws): products against the oracle where the work of an
output tile is shared by several blocks, the fixed-order fix-up (bit-identical results run to
run, and in graph replays), the tile counters left at zero for the next call, and agreement
with the whole-tile kernel (awq_gemm_bits) to fp32 rounding."""
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


def _counters(ws, M, N):
    # the workspace's tile counters: one int32 per 64-row x 128-column tile, after the 2 x 256
    # partial tiles of 128 x 128 fp32
    off = 2 * 256 * 128 * 128 * 4
    return ws[off:off + (M + 63) // 64 * ((N + 127) // 128) * 4].view(torch.int32)


def _sampled(N, seed):
    if N <= 300:
        return np.arange(N)
    g = np.random.default_rng(seed)
    return np.union1d(g.choice(N, size=160, replace=False), np.arange(N - 40, N))


@pytest.mark.parametrize("M,N,K,bits", [
    (33, 2048, 16384, 4),   # 8 groups per block: 16 blocks share each tile
    (37, 2000, 16384, 4),   # ragged M and N
    (64, 8192, 8192, 4),    # two or three blocks per tile
    (100, 2048, 16384, 4),  # two row tiles
    (256, 4096, 4096, 4),   # 64-row tiles at M = 256
    (255, 1000, 28672, 4),  # 128-row tiles, two stages (long K)
    (40, 4000, 16384, 3),
    (129, 3000, 8192, 3),
])
def test_streamk_parity(M, N, K, bits):
    note(f"stream-K M={M} N={N} K={K} bits={bits}")
    assert awq.awq_gemm_kernel(M, N, K, bits=bits).endswith("stream-K")
    seed = 31 * M + N + K + bits
    q, z, sc, p, scd, zd = (_random_packed3 if bits == 3 else _random_packed)(N, K, seed=seed)
    x = activations_fp16(M, K, seed=seed + 1)
    y = host(awq.awq_gemm(dev(x), p, scd, zd))
    rows = _sampled(N, seed + 2)
    assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"stream-K M={M} N={N} K={K}")
    # every row of the split product agrees with the whole-tile kernel to fp32 rounding
    y0 = host(awq.awq_gemm(dev(x), p, scd, zd, workspace=None))
    assert_y_close(y, y0.astype(np.float64), "stream-K against whole tiles")


def test_streamk_deterministic_and_counters_reset():
    """Two calls on one workspace give the same bits (the fix-up adds the parts in the order of
    their K ranges, whichever block finishes last), and leave the tile counters at zero."""
    M, N, K = 48, 4096, 8192
    note(f"stream-K determinism M={M} N={N} K={K}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=401)
    x = dev(activations_fp16(M, K, seed=402))
    nb = awq.awq_gemm_workspace_bytes(M, N, K)
    assert nb > 0
    ws = torch.zeros(nb, dtype=torch.uint8, device=x.device)
    a = host(awq.awq_gemm(x, p, scd, zd, workspace=ws))
    cnt = _counters(ws, M, N)
    assert int(cnt.abs().sum()) == 0
    b = host(awq.awq_gemm(x, p, scd, zd, workspace=ws))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert int(cnt.abs().sum()) == 0


def test_streamk_workspace_shared_by_sizes():
    """One cleared workspace serves calls of different sizes in any order: the partials of one
    call never land where another call's counters are."""
    ws = None
    cases = [(64, 8192, 8192), (33, 2048, 16384), (256, 4096, 4096), (48, 4096, 8192)]
    packs = {}
    for M, N, K in cases + cases[::-1]:
        note(f"stream-K shared workspace M={M} N={N} K={K}")
        if (N, K) not in packs:
            packs[(N, K)] = _random_packed(N, K, seed=N + K)
        q, z, sc, p, scd, zd = packs[(N, K)]
        nb = awq.awq_gemm_workspace_bytes(M, N, K)
        if ws is None or ws.numel() < nb:
            big = max(awq.awq_gemm_workspace_bytes(*c) for c in cases)
            ws = torch.zeros(big, dtype=torch.uint8, device="cuda:0")
        x = activations_fp16(M, K, seed=M + K)
        y = host(awq.awq_gemm(dev(x), p, scd, zd, workspace=ws))
        rows = _sampled(N, M)
        assert_y_close(y[:, rows], oracle.gemm(x, q[rows], z[rows], sc[rows]), f"shared ws M={M} N={N} K={K}")
        assert int(_counters(ws, M, N).abs().sum()) == 0


def test_streamk_graph_replays():
    """The split product captured in a HIP graph: every replay (with eager work and
    synchronizations in between) equals the eager result bit for bit."""
    M, N, K = 64, 8192, 8192
    note(f"stream-K graph M={M} N={N} K={K}")
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=403)
    x = dev(activations_fp16(M, K, seed=404))
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    ref = host(awq.awq_gemm(x, p, scd, zd))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        awq.awq_gemm(x, p, scd, zd, out=y)  # allocates the stream's workspace outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        awq.awq_gemm(x, p, scd, zd, out=y)
    for i in range(3):
        y.zero_()
        g.replay()
        got = host(y)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), f"replay {i}"
        host(awq.awq_gemm(x, p, scd, zd))  # eager work between replays


def test_streamk_workspace_errors():
    M, N, K = 64, 8192, 8192
    q, z, sc, p, scd, zd = _random_packed(N, K, seed=405)
    x = dev(activations_fp16(M, K, seed=406))
    nb = awq.awq_gemm_workspace_bytes(M, N, K)
    small = torch.zeros(nb - 256, dtype=torch.uint8, device=x.device)
    with pytest.raises(awq.AwqError):
        awq.awq_gemm(x, p, scd, zd, workspace=small)
    # no split for M <= 32: no workspace needed, and a given one is not touched
    assert awq.awq_gemm_workspace_bytes(32, N, K) == 0
    ws = torch.full((4096,), 7, dtype=torch.uint8, device=x.device)
    x32 = dev(activations_fp16(32, K, seed=407))
    y = host(awq.awq_gemm(x32, p, scd, zd, workspace=ws))
    assert np.array_equal(y.view(np.uint16), host(awq.awq_gemm(x32, p, scd, zd, workspace=None)).view(np.uint16))
    assert bool((ws == 7).all())
