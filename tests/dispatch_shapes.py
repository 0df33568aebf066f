"""One product shape per kernel the dispatch of awq_gemm_bits (and of awq_gemm_ws) can launch.

Each entry is (kernel, (M, N, K, bits)): awq_gemm_kernel(M, N, K, bits) names that kernel
(its template arguments; block and grid depend on the shape).  tests/test_dispatch.py checks
on the CPU that the dispatch reaches no kernel outside this list over SEARCH_GRID and that
every entry still selects its kernel; tests/test_gpu_dispatch.py runs every entry on the GPU
against the oracle.  Template arguments: gemv_kernel / gemv3_kernel <M, rows per block>;
ring_kernel <bits, 16-row weight tiles per block, groups per stage, stages, x rows staged>;
skinny_kernel <weight tiles per wave, groups per batch, 16-row x tiles>; gemm_pipe_kernel
<x tile rows, stages, LDS bytes, channel sets, waves along N, bits>; gemm_kernel <bits>."""

BRANCHES = [
    ("gemv_kernel<1,4>", (1, 64, 128, 4)),
    ("gemv_kernel<1,8>", (1, 8192, 8192, 4)),
    ("gemv_kernel<2,4>", (2, 64, 128, 4)),
    ("gemv_kernel<2,8>", (2, 16384, 128, 4)),
    ("gemv3_kernel<1,4>", (1, 64, 128, 3)),
    ("gemv3_kernel<1,8>", (1, 8192, 8192, 3)),
    ("gemv3_kernel<2,4>", (2, 64, 128, 3)),
    ("gemv3_kernel<2,8>", (2, 16384, 128, 3)),
    ("ring_kernel<4,1,1,2,4>", (3, 64, 128, 4)),
    ("ring_kernel<4,1,1,2,8>", (5, 64, 128, 4)),
    ("ring_kernel<4,2,1,2,8>", (5, 16384, 128, 4)),
    ("ring_kernel<4,4,1,2,8>", (5, 16384, 8192, 4)),
    ("ring_kernel<4,1,1,2,16>", (9, 64, 128, 4)),
    ("ring_kernel<4,2,1,2,16>", (9, 16384, 128, 4)),
    ("ring_kernel<4,4,1,2,16>", (9, 8200, 8192, 4)),
    ("ring_kernel<4,1,1,2,32>", (17, 64, 128, 4)),
    ("ring_kernel<4,2,1,2,32>", (17, 64, 16384, 4)),
    ("ring_kernel<4,4,1,2,32>", (17, 12300, 8192, 4)),
    ("ring_kernel<4,1,1,2,64>", (33, 64, 128, 4)),
    ("ring_kernel<4,2,1,2,64>", (33, 8200, 8192, 4)),
    ("ring_kernel<3,1,1,2,4>", (3, 64, 128, 3)),
    ("ring_kernel<3,1,1,2,8>", (5, 64, 128, 3)),
    ("ring_kernel<3,2,1,2,8>", (5, 16384, 128, 3)),
    ("ring_kernel<3,4,1,2,8>", (5, 16384, 8192, 3)),
    ("ring_kernel<3,1,1,2,16>", (9, 64, 128, 3)),
    ("ring_kernel<3,2,1,2,16>", (9, 16384, 128, 3)),
    ("ring_kernel<3,4,1,2,16>", (9, 8200, 8192, 3)),
    ("ring_kernel<3,1,1,2,32>", (17, 64, 128, 3)),
    ("ring_kernel<3,2,1,2,32>", (17, 64, 16384, 3)),
    ("ring_kernel<3,4,1,2,32>", (17, 12300, 8192, 3)),
    ("ring_kernel<3,1,1,2,64>", (33, 64, 128, 3)),
    ("ring_kernel<3,2,1,2,64>", (33, 8200, 4224, 3)),
    ("skinny_kernel<2,4,1>", (1, 64, 32896, 4)),
    ("skinny_kernel<2,1,2>", (17, 64, 139264, 4)),
    ("skinny_kernel<2,1,3>", (33, 64, 139264, 4)),
    ("skinny_kernel<2,1,4>", (64, 64, 139264, 4)),
    ("gemm_pipe_kernel<64,4,163840,2,4,4>", (65, 64, 128, 4)),
    ("gemm_pipe_kernel<64,3,163840,1,2,4>", (33, 8200, 28672, 4)),
    ("gemm_pipe_kernel<128,3,163840,2,4,4>", (65, 16400, 128, 4)),
    ("gemm_pipe_kernel<128,2,163840,1,4,4>", (65, 64, 28672, 4)),
    ("gemm_pipe_kernel<64,4,163840,2,4,3>", (65, 64, 128, 3)),
    ("gemm_pipe_kernel<128,3,163840,2,4,3>", (65, 16400, 128, 3)),
    ("gemm_kernel<4>", (65, 64, 32896, 4)),
    ("gemm_kernel<3>", (1, 64, 32896, 3)),
]

# The same kernels where awq_gemm_ws (a workspace given) splits their work over the compute
# units (stream-K): awq_gemm_ws_kernel names the kernel and ends in "stream-K".
STREAMK_BRANCHES = [
    ("gemm_pipe_kernel<64,4,163840,2,4,4>", (37, 2000, 16384, 4)),
    ("gemm_pipe_kernel<64,3,163840,1,2,4>", (33, 4096, 28672, 4)),
    ("gemm_pipe_kernel<128,2,163840,1,4,4>", (200, 1000, 32768, 4)),
    ("gemm_pipe_kernel<128,3,163840,2,4,4>", (256, 16400, 1024, 4)),
    ("gemm_pipe_kernel<64,4,163840,2,4,3>", (40, 4000, 16384, 3)),
    ("gemm_pipe_kernel<128,3,163840,2,4,3>", (256, 16400, 1024, 3)),
]

# Sizes whose products the coverage check enumerates (both code widths): every M class of the
# dispatch, row counts around its bounds (8192, 12288, 16384) and the model shapes, K from one
# group to past every LDS limit.
SEARCH_GRID = dict(
    M=[1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 20, 24, 32, 33, 40, 48, 64, 65, 100, 128, 256, 1024, 5000],
    N=[1, 64, 100, 300, 4096, 8192, 8200, 10240, 12288, 12300, 16384, 16400, 22016, 28672],
    K=[128, 512, 1024, 4096, 4224, 6144, 8192, 11008, 16384, 16640, 28672, 32768, 32896, 36096, 65536,
       139264, 270336, 524288, 1048576],
)
