"""The measurement kernel that bounds the decode GEMV's shape (libawq_ceilings.so): the read
that ends every block with one dependent store really reads every byte it is given.  Each
block's stored word must equal the XOR of all 32-bit words of the 16-byte pieces its threads
loaded, computed on the host (threads past the end reload the last piece)."""
import ctypes
import os

import numpy as np
import pytest
import torch

from test_gpu_parity import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_quantization_gemm_amd", "libawq_ceilings.so"))
    f = lib.awq_ceiling_stream_read_store
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("nbytes", [1 << 20, (1 << 20) + 48, 4096 * 3 + 16])
@pytest.mark.parametrize("L", [1, 2, 4])
def test_stream_read_store_folds_every_piece(nbytes, L):
    note(f"ceiling read+store bytes={nbytes} L={L}")
    f = _lib()
    g = np.random.default_rng(nbytes + L)
    words = g.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).to("cuda:0")
    n16 = nbytes // 16
    blocks = -(-n16 // (256 * L))
    out = torch.full((blocks + 1,), -1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert f(src.data_ptr(), nbytes, out.data_ptr(), blocks, L, st) == 0
    assert f(src.data_ptr(), nbytes, out.data_ptr(), blocks - 1, L, st) == 1  # too few output words
    got = out.cpu().numpy().view(np.uint32)
    piece = np.bitwise_xor.reduce(words.reshape(n16, 4), axis=1)
    for b in range(blocks):
        idx = np.minimum(np.arange(b * 256 * L, (b + 1) * 256 * L), n16 - 1)
        assert got[b] == np.bitwise_xor.reduce(piece[idx]), f"block {b}"
    assert got[blocks] == np.uint32(0xFFFFFFFF)  # nothing past the blocks' words
