"""The C ABI on the host: every declared symbol is exported, size queries match the
documented format (and the pages' memory figures), and bad arguments are refused
with the documented status before anything is launched (no GPU needed)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest
import torch

import weight_only_quantization_gemm_amd as awq
from weight_only_quantization_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

OK, INVALID, MISALIGNED, WS_SMALL = 0, 1, 2, 3
FAKE = 0x10000          # aligned, non-null; never dereferenced because validation fails first
FAKE_MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("awq_quantize", "awq_gemm", "awq_pack", "awq_unpack", "awq_channel_mean_abs"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_ceilings_library_exports_and_refuses_bad_arguments():
    """libawq_ceilings.so (the measurement kernels bench.py compares against) exports what
    include/awq_ceilings.h declares and refuses bad arguments before launching."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "awq_ceilings.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(awq_ceiling_[a-z0-9_]+)\s*\(", text)))
    assert names == ["awq_ceiling_mfma_f16", "awq_ceiling_stream_read", "awq_ceiling_stream_read_store"]
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_quantization_gemm_amd", "libawq_ceilings.so"))
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    f = lib.awq_ceiling_stream_read_store
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    nb = 1 << 20  # 256 blocks at one load per thread, 128 at two
    assert f(FAKE, nb, FAKE, 255, 1, None) == INVALID       # out holds fewer words than blocks
    assert f(FAKE, nb, FAKE, 128, 3, None) == INVALID       # loads per thread not 1, 2 or 4
    assert f(FAKE_MISALIGNED, nb, FAKE, 256, 1, None) == INVALID
    assert f(FAKE, nb, FAKE_MISALIGNED, 256, 1, None) == INVALID
    assert f(FAKE, nb + 8, FAKE, 257, 1, None) == INVALID  # bytes not a multiple of 16
    assert f(None, nb, FAKE, 256, 1, None) == INVALID


def test_version_and_status_strings():
    assert awq.awq_version() >= 10000
    assert awq.awq_status_string(0) == "AWQ_OK"
    assert awq.awq_status_string(3) == "AWQ_ERROR_WORKSPACE_TOO_SMALL"
    assert awq.awq_status_string(99) == "AWQ_UNKNOWN_STATUS"


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (4096, 4096), (4096, 11008), (28672, 8192)])
def test_size_queries(N, K):
    G = K // 128
    assert awq.awq_packed_bytes(N, K) == N * K // 2
    assert awq.awq_scales_bytes(N, K) == 2 * N * G
    assert awq.awq_zeros_bytes(N, K) == N * ((G + 1) // 2)
    assert awq.awq_packed_bytes(N, K + 4) == 0  # K % 8 != 0
    assert awq.awq_scales_bytes(N, K + 8) == 0  # K % group != 0


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (4096, 4096), (4096, 11008), (28672, 8192)])
def test_size_queries_three_bit(N, K):
    assert awq.awq_packed_bytes(N, K, bits=3) == 3 * N * K // 8
    assert _lib.load().awq_packed_bytes_bits(N, K, 4) == N * K // 2
    assert _lib.load().awq_packed_bytes_bits(N, K, 5) == 0
    assert _lib.load().awq_packed_bytes_bits(N, K + 16, 3) == 0  # K % 32 != 0
    assert awq.packed_words(K, 3) * 4 * N == awq.awq_packed_bytes(N, K, bits=3)


def test_byte_accounting_matches_page_figures():
    figs = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    N, K = 4096, 4096
    fp16_bytes = 2 * N * K
    codes = awq.awq_packed_bytes(N, K)
    meta = awq.awq_scales_bytes(N, K) + awq.awq_zeros_bytes(N, K)
    # the codes alone are exactly a quarter of fp16 weights; with group metadata
    # 4.156 bits per weight, still "about a quarter" (within 5%)
    assert codes / fp16_bytes == figs["weight_memory_fraction_4bit"]["value"]
    assert abs((codes + meta) / fp16_bytes - 0.25) / 0.25 < 0.05
    assert abs(8 * (codes + meta) / (N * K) - 4.15625) < 1e-12
    assert abs(fp16_bytes / (codes + meta) - figs["decode_traffic_reduction"]["value"]) / 4.0 < 0.05


def test_workspace_query():
    assert awq.awq_quantize_workspace_bytes(512, 512, 64, 128, 20) > 0
    assert awq.awq_quantize_workspace_bytes(512, 500, 64, 128, 20) == 0
    assert awq.awq_quantize_workspace_bytes(512, 512, 64, 64, 20) == 0
    assert awq.awq_quantize_workspace_bytes(512, 512, 64, 128, 65) == 0
    # Gram form (M >= K): X^T fp16, G fp32 + fp16 hi/lo, E' fp16 hi/lo
    big = awq.awq_quantize_workspace_bytes(4096, 11008, 65536, 128, 20)
    assert big >= 2 * 11008 * 65536 + 8 * 11008 * 11008 + 4 * 4096 * 11008
    # direct form (M < K): E in fp32, no Gram buffers; s (fp32) and 1/s (fp64) per alpha
    small = awq.awq_quantize_workspace_bytes(4096, 11008, 64, 128, 20)
    assert 4 * 4096 * 11008 + 12 * 20 * 11008 <= small < 4 * 4096 * 11008 + 12 * 20 * 11008 + (1 << 20)


def _lib_():
    return _lib.load()


def test_gemm_argument_errors_before_launch():
    lib = _lib_()
    f = lib.awq_gemm
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, None) == INVALID
    assert "NULL" in awq.awq_last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 100, 128, None) == INVALID    # K % group
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 64, None) == INVALID     # group
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 128, 128, None) == INVALID    # M
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 128, 128, None) == INVALID     # N
    assert f(FAKE_MISALIGNED, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, None) == MISALIGNED


def test_input_scaling_queries_and_errors_before_launch():
    lib = _lib_()
    ws = lib.awq_gemm_scaled_workspace_bytes
    assert ws(1, 4096, 4096, 4) == 4096 * 2 and ws(2, 300, 16384, 4) == 2 * 16384 * 2
    assert ws(3, 64, 4096, 4) == 3 * 4096 * 2 and ws(1, 64, 4096, 3) == 4096 * 2
    assert ws(5, 64, 136, 4) == (5 * 136 * 2 + 255) // 256 * 256
    assert ws(0, 64, 4096, 4) == 0 and ws(1, 64, 4096, 5) == 0
    assert lib.awq_scale_input(FAKE, FAKE, 1, 12, FAKE, None) == INVALID       # K % 8
    assert lib.awq_scale_input(FAKE, FAKE, 0, 128, FAKE, None) == INVALID
    assert lib.awq_scale_input(FAKE, None, 1, 128, FAKE, None) == INVALID
    f = lib.awq_gemm_scaled
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, 4, FAKE, 256, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, 4, None, 256, None) == INVALID   # workspace
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 100, 128, 4, FAKE, 256, None) == INVALID   # K % group
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, 5, FAKE, 256, None) == INVALID   # bits
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 64, 128, 128, 4, FAKE, 767, None) == WS_SMALL
    assert "workspace" in awq.awq_last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 64, 128, 128, 4, FAKE_MISALIGNED, 768, None) == MISALIGNED
    assert "workspace" in awq.awq_last_error()


# Every device pointer of every entry point, by argument position: a call that is valid
# except for that one pointer being 8 bytes off a 16-byte boundary must return
# AWQ_ERROR_MISALIGNED and name the pointer (so no kernel ever sees it).
_AL = np.arange(20, dtype=np.float32) / np.float32(20)
_WS_Q = 1 << 40
MISALIGNED_CASES = {
    "awq_channel_mean_abs": ((FAKE, 64, 256, FAKE, None), {0: "X", 3: "a"}),
    "awq_pack_bits": ((FAKE, FAKE, 64, 256, 128, 4, FAKE, FAKE, FAKE, None),
                      {0: "W", 1: "s", 6: "packed", 7: "scales", 8: "zeros"}),
    "awq_quantize_shared": ((FAKE, FAKE, 64, 256, 32, 128, 4, _AL.ctypes.data, 20, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, _WS_Q, None),
                            {0: "W", 1: "X", 10: "packed", 11: "scales", 12: "zeros", 13: "s", 14: "best_alpha",
                             15: "loss", 16: "workspace"}),
    "awq_keep_fp16_ablation": ((FAKE, FAKE, 64, 256, 32, 128, 4, 3, FAKE, FAKE, FAKE, FAKE, FAKE, _WS_Q, None),
                               {0: "W", 1: "X", 8: "random_keep", 9: "keep_act", 10: "keep_wt", 11: "loss",
                                12: "workspace"}),
    "awq_gemm_bits": ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 256, 128, 4, None),
                      {0: "x", 1: "packed", 2: "scales", 3: "zeros", 4: "y"}),
    "awq_scale_input": ((FAKE, FAKE, 1, 256, FAKE, None), {0: "x", 1: "s", 4: "xs"}),
    "awq_gemm_scaled": ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 64, 256, 128, 4, FAKE, 1 << 20, None),
                        {0: "x", 1: "s", 2: "packed", 3: "scales", 4: "zeros", 5: "y", 11: "workspace"}),
    "awq_unpack_bits": ((FAKE, FAKE, 64, 256, 128, 4, FAKE, FAKE, None),
                        {0: "packed", 1: "zeros", 6: "codes", 7: "zeros_u8"}),
}


@pytest.mark.parametrize("entry", sorted(MISALIGNED_CASES))
def test_every_device_pointer_is_alignment_checked(entry):
    lib = _lib_()
    fn = getattr(lib, entry)
    args, pointers = MISALIGNED_CASES[entry]
    for pos, name in pointers.items():
        bad = list(args)
        bad[pos] = FAKE_MISALIGNED
        assert fn(*bad) == MISALIGNED, f"{entry}: {name} at argument {pos}"
        assert awq.awq_last_error() == f"{name} must be 16-byte aligned", (entry, awq.awq_last_error())


def test_misaligned_case_table_covers_every_pointer_argument():
    """The table above names every pointer parameter the header declares for these entry
    points (host pointers excepted: the alpha grid and the stream)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for entry, (args, pointers) in MISALIGNED_CASES.items():
        decl = re.search(entry + r"\s*\(([^;]*)\)\s*;", text).group(1)
        params = [p.strip() for p in decl.split(",")]
        assert len(params) == len(args), entry
        ptr_params = {i for i, p in enumerate(params) if "*" in p and not p.endswith(("alphas", "stream"))}
        assert ptr_params == set(pointers), (entry, sorted(ptr_params), sorted(pointers))
        for i, name in pointers.items():
            assert re.search(r"\b" + name + r"$", params[i]), (entry, i, params[i])


def test_quantize_shared_argument_errors_before_launch():
    lib = _lib_()
    al = (ctypes.c_float * 2)(0.0, 0.5)
    f = lib.awq_quantize_shared
    args = lambda reuse, ws=FAKE, wsb=1 << 40: (FAKE, FAKE, 64, 512, 600, 128, 4, ctypes.cast(al, ctypes.c_void_p), 2,
                                                reuse, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, wsb, None)
    assert f(*args(2)) == INVALID
    assert f(*args(-1)) == INVALID
    assert f(*args(1, wsb=16)) == WS_SMALL


def test_pack_and_unpack_argument_errors_before_launch():
    lib = _lib_()
    assert lib.awq_pack(None, None, 4, 128, 128, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.awq_pack(FAKE, None, 4, 130, 128, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.awq_pack(FAKE, FAKE_MISALIGNED, 4, 128, 128, FAKE, FAKE, FAKE, None) == MISALIGNED
    assert lib.awq_unpack(FAKE, FAKE, 4, 128, 32, FAKE, FAKE, None) == INVALID
    assert lib.awq_channel_mean_abs(FAKE, 0, 128, FAKE, None) == INVALID
    assert lib.awq_channel_mean_abs(FAKE, (1 << 23) + 1, 128, FAKE, None) == INVALID
    assert lib.awq_channel_mean_abs(FAKE, 4, 12, FAKE, None) == INVALID
    assert lib.awq_channel_mean_abs(FAKE_MISALIGNED, 4, 16, FAKE, None) == MISALIGNED


def test_bits_argument_errors_before_launch():
    lib = _lib_()
    for bits in (0, 2, 5, 8):
        assert lib.awq_pack_bits(FAKE, None, 4, 128, 128, bits, FAKE, FAKE, FAKE, None) == INVALID
        assert "bits" in awq.awq_last_error()
        assert lib.awq_gemm_bits(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, bits, None) == INVALID
        assert lib.awq_unpack_bits(FAKE, FAKE, 4, 128, 128, bits, FAKE, FAKE, None) == INVALID
    al = np.arange(20, dtype=np.float32) / np.float32(20)
    ws = awq.awq_quantize_workspace_bytes(64, 256, 32, 128, 20)
    assert lib.awq_quantize_bits(FAKE, FAKE, 64, 256, 32, 128, 2, al.ctypes.data, 20, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None, FAKE, ws, None) == INVALID
    assert lib.awq_gemm_bits(FAKE_MISALIGNED, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, 3, None) == MISALIGNED


def test_gemm_ws_argument_errors_before_launch():
    """awq_gemm_ws: the workspace size query is 0 where the GEMM splits no work (and for bad
    sizes), a needed workspace must be given, large enough and 16-byte aligned, and the other
    arguments are checked as for awq_gemm_bits."""
    lib = _lib_()
    f = lib.awq_gemm_ws
    M, N, K = 64, 8192, 8192  # split: 64 tiles of 64 groups over 256 compute units
    nb = lib.awq_gemm_workspace_bytes(M, N, K, 4)
    assert nb > 0 and nb % 256 == 0
    assert lib.awq_gemm_workspace_bytes(M, N, K, 3) == nb
    for bad in ((0, N, K, 4), (M, 0, K, 4), (M, N, 100, 4), (M, N, K, 2), (32, N, K, 4), (1, N, K, 4)):
        assert lib.awq_gemm_workspace_bytes(*bad) == 0, bad
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, 128, 4, None, 0, None) == INVALID
    assert "workspace" in awq.awq_last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, 128, 4, FAKE, nb - 256, None) == WS_SMALL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, 128, 4, FAKE_MISALIGNED, nb, None) == MISALIGNED
    for pos in range(5):
        args = [FAKE] * 5
        args[pos] = FAKE_MISALIGNED
        assert f(*args, M, N, K, 128, 4, FAKE, nb, None) == MISALIGNED, pos
        args[pos] = None
        assert f(*args, M, N, K, 128, 4, FAKE, nb, None) == INVALID, pos
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, 128, 5, FAKE, nb, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, 100, 128, 4, FAKE, nb, None) == INVALID
    buf = ctypes.create_string_buffer(160)
    assert lib.awq_gemm_ws_kernel(M, N, K, 128, 4, buf, 160) == OK
    assert buf.value.decode().endswith("stream-K")
    assert lib.awq_gemm_ws_kernel(16, N, K, 128, 4, buf, 160) == OK
    assert not buf.value.decode().endswith("stream-K")


def test_ablation_argument_errors_before_launch():
    lib = _lib_()
    f = lib.awq_keep_fp16_ablation
    ws = awq.awq_ablation_workspace_bytes(64, 256, 32)
    assert ws >= awq.awq_quantize_workspace_bytes(64, 256, 32, 128, 1) + 9 * 256 > 0
    base = dict(W=FAKE, X=FAKE, N=64, K=256, M=32, g=128, bits=4, nk=3, rk=FAKE, ka=FAKE, kw=FAKE, loss=FAKE,
                ws=FAKE, wsb=ws, st=None)
    call = lambda **kw: f(*dict(base, **kw).values())
    assert call(nk=257) == INVALID and "n_keep" in awq.awq_last_error()
    assert call(nk=-1) == INVALID
    assert call(rk=None) == INVALID
    assert call(bits=2) == INVALID
    assert call(M=0) == INVALID
    assert call(N=(1 << 23) + 1) == INVALID
    assert call(wsb=ws - 1) == WS_SMALL
    assert call(X=FAKE_MISALIGNED) == MISALIGNED


def test_quantize_argument_errors_before_launch():
    lib = _lib_()
    q = lib.awq_quantize
    al = np.arange(20, dtype=np.float32) / np.float32(20)
    ws = awq.awq_quantize_workspace_bytes(64, 256, 32, 128, 20)
    args = lambda **kw: dict(dict(W=FAKE, X=FAKE, N=64, K=256, M=32, g=128, al=al.ctypes.data, na=20,
                                   packed=FAKE, scales=FAKE, zeros=FAKE, s=FAKE, best=FAKE, loss=None,
                                   ws=FAKE, wsb=ws, st=None), **kw)
    call = lambda d: q(*d.values())
    assert call(args(wsb=ws - 1)) == WS_SMALL
    assert "workspace" in awq.awq_last_error()
    assert call(args(na=0)) == INVALID
    assert call(args(na=65)) == INVALID
    bad = al.copy()
    bad[3] = np.nan
    assert call(args(al=bad.ctypes.data)) == INVALID
    bad[3] = -0.5
    assert call(args(al=bad.ctypes.data)) == INVALID
    assert call(args(M=0)) == INVALID
    assert call(args(X=None)) == INVALID
    assert call(args(ws=FAKE_MISALIGNED)) == MISALIGNED
    assert call(args(K=200)) == INVALID


def test_binding_refuses_cpu_tensors():
    W = torch.zeros((8, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        awq.awq_pack(W)
    with pytest.raises(ValueError, match="GPU"):
        awq.awq_gemm(torch.zeros((1, 128), dtype=torch.float16), torch.zeros((8, 16), dtype=torch.int32),
                     torch.zeros((8, 1), dtype=torch.float16), torch.zeros((8, 1), dtype=torch.uint8))


def test_host_layout_codec_roundtrip():
    from layout import decode_codes, decode_zeros, encode
    g = np.random.default_rng(0)
    for N, K in ((3, 128), (5, 384), (2, 1024)):
        codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
        zeros = g.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
        p, zb = encode(codes, zeros)
        assert np.array_equal(decode_codes(p, K), codes)
        assert np.array_equal(decode_zeros(zb, K // 128), zeros)
    # word layout: channel 8w+1 lives in nibble 4, channel 8w+2 in nibble 1
    c = np.zeros((1, 128), np.uint8)
    c[0, 1] = 0xA
    c[0, 2] = 0x5
    p, _ = encode(c, np.zeros((1, 1), np.uint8))
    assert int(p.view(np.uint32)[0, 0]) == (0xA << 16) | (0x5 << 4)


def test_host_layout_codec_roundtrip_three_bit():
    from layout import decode_codes3, decode_zeros, encode3
    g = np.random.default_rng(1)
    for N, K in ((3, 128), (5, 384), (2, 1024)):
        codes = g.integers(0, 8, size=(N, K)).astype(np.uint8)
        zeros = g.integers(0, 8, size=(N, K // 128)).astype(np.uint8)
        p, zb = encode3(codes, zeros)
        assert p.shape == (N, 3 * K // 32)
        assert np.array_equal(decode_codes3(p, K), codes)
        assert np.array_equal(decode_zeros(zb, K // 128), zeros)
    # word placement worked out from the format statement: channel 2 (pair 1, even) in
    # bits 3..5 of word 0; channel 11 (pair 5: word 1, field 0, odd) in bits 16..18 of
    # word 1; code 6 = 0b110 of channel 30 sets bit 15 of words 1 and 2; code 4 of
    # channel 31 sets bit 31 of word 2.
    c = np.zeros((1, 128), np.uint8)
    c[0, 2], c[0, 11], c[0, 30], c[0, 31] = 5, 3, 6, 4
    p, _ = encode3(c, np.zeros((1, 1), np.uint8))
    w = p.view(np.uint32)[0, :3]
    assert int(w[0]) == 5 << 3
    assert int(w[1]) == (3 << 16) | (1 << 15)
    assert int(w[2]) == (1 << 15) | (1 << 31)
