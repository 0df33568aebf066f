"""awq_gemm_scaled_static, the entry point that allocates nothing, against awq_gemm_scaled.

Both go through the C ABI.  Two calls in a row on one stream, the second on a smaller input
than the first, each compared bit for bit with awq_gemm_scaled (workspace from the caller) and
with the oracle's product on x / s to the product bars; then a call whose scaled input would
exceed the static array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16
from layout import assert_y_close
from weight_only_quantization_gemm_amd import _lib

pytestmark = pytest.mark.gpu

dev0 = torch.device("cuda:0")


def _scales(K, seed):
    g = np.random.default_rng(seed)
    return oracle.scales_for_alpha(np.exp(g.normal(0.0, 0.8, K)), 0.5)


def _layer(N, K, bits, seed):
    from test_gpu_parity import _random_packed
    from test_gpu_three_bit import _random_packed3
    return (_random_packed if bits == 4 else _random_packed3)(N, K, seed=seed)


def _static(x, s, p, sc, z, y, M, N, K, bits):
    lib = _lib.load()
    st = torch.cuda.current_stream(dev0).cuda_stream
    return lib.awq_gemm_scaled_static(x.data_ptr(), s.data_ptr(), p.data_ptr(), sc.data_ptr(), z.data_ptr(),
                                      y.data_ptr(), M, N, K, 128, bits, st)


def _scaled(x, s, p, sc, z, y, M, N, K, bits):
    lib = _lib.load()
    need = lib.awq_gemm_scaled_workspace_bytes(M, N, K, bits)
    ws = torch.empty(need, dtype=torch.uint8, device=dev0)
    st = torch.cuda.current_stream(dev0).cuda_stream
    rc = lib.awq_gemm_scaled(x.data_ptr(), s.data_ptr(), p.data_ptr(), sc.data_ptr(), z.data_ptr(), y.data_ptr(),
                             M, N, K, 128, bits, ws.data_ptr(), need, st)
    return rc, ws


@pytest.mark.parametrize("bits", [4, 3])
def test_static_scratch_matches_workspace_path(bits):
    cases = [(300, 1000, 4096), (2, 4096, 1024)]  # the second call smaller than the first
    keep = []
    for i, (M, N, K) in enumerate(cases):
        print(f"no-alloc gemm_scaled call {i}: M={M} N={N} K={K} bits={bits}", flush=True)
        q, z, sc, p, scd, zd = _layer(N, K, bits, seed=100 * i + bits)
        s = _scales(K, 7 + i)
        x = activations_fp16(M, K, seed=11 + i)
        xd, sd = torch.from_numpy(x).to(dev0), torch.from_numpy(s).to(dev0)
        y_static = torch.empty((M, N), dtype=torch.float16, device=dev0)
        y_ws = torch.empty_like(y_static)
        assert _static(xd, sd, p, scd, zd, y_static, M, N, K, bits) == 0, awq.awq_last_error()
        rc, ws = _scaled(xd, sd, p, scd, zd, y_ws, M, N, K, bits)
        assert rc == 0, awq.awq_last_error()
        torch.cuda.synchronize()
        a, b = y_static.cpu().numpy(), y_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"call {i}"
        assert_y_close(a, oracle.gemm(oracle.scaled_input(x, s), q, z, sc), f"call {i} bits={bits}")
        keep.append(ws)


def test_static_scratch_refuses_oversized_input():
    lib = _lib.load()
    fake = 0x10000
    M, K = 2049, 4096  # 2049 * 4096 * 2 bytes > 16 MiB
    rc = lib.awq_gemm_scaled_static(fake, fake, fake, fake, fake, fake, M, 64, K, 128, 4, None)
    assert rc == 1 and "static scratch" in awq.awq_last_error()
