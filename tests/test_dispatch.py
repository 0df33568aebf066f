"""The product dispatch, checked on the CPU through awq_gemm_kernel (a dry run of
awq_gemm_bits's own dispatch that launches nothing): over a broad grid of sizes it reaches
no kernel that tests/dispatch_shapes.py does not list, and every listed shape still selects
its kernel, so tests/test_gpu_dispatch.py runs each kernel the product can launch."""
import itertools

import pytest

import weight_only_quantization_gemm_amd as awq
from dispatch_shapes import BRANCHES, SEARCH_GRID, STREAMK_BRANCHES


def _kernel(M, N, K, bits):
    """The kernel awq_gemm_bits (no workspace: whole output tiles) launches."""
    return awq.awq_gemm_kernel(M, N, K, bits=bits, workspace=False).split(" ")[0]


def test_listed_shapes_select_their_kernel():
    for name, (M, N, K, bits) in BRANCHES:
        assert _kernel(M, N, K, bits) == name, (name, (M, N, K, bits))
    assert len({n for n, _ in BRANCHES}) == len(BRANCHES)


def test_dispatch_reaches_only_listed_kernels():
    listed = {n for n, _ in BRANCHES}
    reached = {}
    for bits in (4, 3):
        for M, N, K in itertools.product(SEARCH_GRID["M"], SEARCH_GRID["N"], SEARCH_GRID["K"]):
            reached.setdefault(_kernel(M, N, K, bits), (M, N, K, bits))
    missing = {k: v for k, v in reached.items() if k not in listed}
    assert not missing, f"kernels without a parity shape: {missing}"
    unreached = listed - set(reached)
    assert not unreached, f"listed kernels the grid no longer reaches: {unreached}"


def test_streamk_reaches_only_listed_kernels():
    """With a workspace the dispatch is the same except where the GEMM splits its work: those
    kernels (texts ending in "stream-K") are the listed stream-K branches, and the workspace
    size query is positive exactly there."""
    listed = {n for n, _ in STREAMK_BRANCHES}
    for name, (M, N, K, bits) in STREAMK_BRANCHES:
        text = awq.awq_gemm_kernel(M, N, K, bits=bits, workspace=True)
        assert text.split(" ")[0] == name and text.endswith("stream-K"), (name, text)
    reached = {}
    for bits in (4, 3):
        for M, N, K in itertools.product(SEARCH_GRID["M"], SEARCH_GRID["N"], SEARCH_GRID["K"]):
            text = awq.awq_gemm_kernel(M, N, K, bits=bits, workspace=True)
            split = text.endswith("stream-K")
            assert split == (awq.awq_gemm_workspace_bytes(M, N, K, bits) > 0), (M, N, K, bits, text)
            if split:
                reached.setdefault(text.split(" ")[0], (M, N, K, bits))
                assert M > 32
            else:
                assert text == awq.awq_gemm_kernel(M, N, K, bits=bits, workspace=False)
    missing = {k: v for k, v in reached.items() if k not in listed}
    assert not missing, f"stream-K kernels without a parity shape: {missing}"
    assert listed == set(reached)


def test_dispatch_by_m_class():
    # the decode GEMV below M = 3 (M = 2 up to K = 16384), matrix-core kernels above
    assert _kernel(1, 4096, 4096, 4).startswith("gemv_kernel<1,")
    assert _kernel(2, 4096, 4096, 4).startswith("gemv_kernel<2,")
    assert _kernel(2, 4096, 16384, 4).startswith("ring_kernel<4,")
    assert _kernel(16, 11008, 4096, 4).startswith("ring_kernel<4,")
    assert _kernel(256, 11008, 4096, 4) == "gemm_pipe_kernel<128,3,163840,2,4,4>"
    assert _kernel(64, 11008, 4096, 4) == "gemm_pipe_kernel<64,4,163840,2,4,4>"


def test_dispatch_query_errors():
    with pytest.raises(awq.AwqError):
        awq.awq_gemm_kernel(1, 100, 100)  # K not a multiple of the group
    with pytest.raises(awq.AwqError):
        awq.awq_gemm_kernel(0, 100, 128)
    with pytest.raises(ValueError):
        awq.awq_gemm_kernel(1, 100, 128, bits=2)
