"""Torch-facing wrappers with the names of the C entry points.

Each wrapper checks dtypes, devices and shapes, allocates outputs with torch on
the input's device, and calls libawq on torch's current stream of that device.
All arithmetic happens in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import AwqError, check, load

GROUP = 128
MAX_ALPHAS = 64
BITS = (4, 3)  # code widths of the packed formats


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libawq has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def default_alpha_grid(n: int = 20) -> np.ndarray:
    """alpha_i = i / n for i = 0..n-1, in float32 (a grid over [0, 1))."""
    return (np.arange(n, dtype=np.float32) / np.float32(n)).astype(np.float32)


# ---------------------------------------------------------------- size queries
def awq_packed_bytes(N: int, K: int, bits: int = 4) -> int:
    return int(load().awq_packed_bytes_bits(N, K, bits))


def awq_scales_bytes(N: int, K: int, group: int = GROUP) -> int:
    return int(load().awq_scales_bytes(N, K, group))


def awq_zeros_bytes(N: int, K: int, group: int = GROUP) -> int:
    return int(load().awq_zeros_bytes(N, K, group))


def awq_quantize_workspace_bytes(N: int, K: int, M: int, group: int = GROUP, n_alpha: int = 20) -> int:
    return int(load().awq_quantize_workspace_bytes(N, K, M, group, n_alpha))


def awq_status_string(status: int) -> str:
    return load().awq_status_string(status).decode()


def awq_last_error() -> str:
    return load().awq_last_error().decode()


def awq_version() -> int:
    return int(load().awq_version())


def _check_bits(bits: int) -> None:
    if bits not in BITS:
        raise ValueError(f"bits must be one of {BITS}, got {bits}")


def packed_words(K: int, bits: int = 4) -> int:
    """int32 words per row of the packed format: K/8 at 4 bits, 3K/32 at 3 bits."""
    _check_bits(bits)
    return K // 8 if bits == 4 else 3 * (K // 32)


def bits_of(packed: torch.Tensor, K: int) -> int:
    """The code width a packed tensor of K input channels was written at (K/8 and 3K/32
    words per row never coincide)."""
    for b in BITS:
        if packed.dim() == 2 and packed.shape[1] == packed_words(K, b):
            return b
    raise ValueError(f"packed {tuple(packed.shape)} matches no format for K={K}")


def empty_packed(N: int, K: int, device, group: int = GROUP, bits: int = 4):
    """Output buffers of the packed format: packed int32 [N][K/8] (4-bit) or [N][3K/32]
    (3-bit), scales fp16 [N][K/g], zeros uint8 [N][ceil(K/g/2)]."""
    G = K // group
    packed = torch.empty((N, packed_words(K, bits)), dtype=torch.int32, device=device)
    scales = torch.empty((N, G), dtype=torch.float16, device=device)
    zeros = torch.empty((N, (G + 1) // 2), dtype=torch.uint8, device=device)
    return packed, scales, zeros


# ---------------------------------------------------------------- entry points
def awq_channel_mean_abs(X: torch.Tensor) -> torch.Tensor:
    _need(X, "X", torch.float16, 2)
    M, K = X.shape
    a = torch.empty((K,), dtype=torch.float64, device=X.device)
    with torch.cuda.device(X.device):
        check(load().awq_channel_mean_abs(X.data_ptr(), M, K, a.data_ptr(), _stream(X.device)))
    return a


def awq_pack(W: torch.Tensor, s: Optional[torch.Tensor] = None, group: int = GROUP, bits: int = 4):
    _need(W, "W", torch.float16, 2)
    _check_bits(bits)
    N, K = W.shape
    if s is not None:
        _need(s, "s", torch.float32, 1)
        if s.shape[0] != K or s.device != W.device:
            raise ValueError("s must be float32 [K] on W's device")
    if K % group:
        raise ValueError(f"K={K} is not a multiple of group {group}")
    packed, scales, zeros = empty_packed(N, K, W.device, group, bits)
    with torch.cuda.device(W.device):
        check(load().awq_pack_bits(W.data_ptr(), _ptr(s), N, K, group, bits, packed.data_ptr(), scales.data_ptr(),
                                   zeros.data_ptr(), _stream(W.device)))
    return packed, scales, zeros


def awq_quantize(W: torch.Tensor, X: torch.Tensor, alphas: Optional[Sequence[float]] = None,
                 group: int = GROUP, workspace: Optional[torch.Tensor] = None, bits: int = 4,
                 reuse_statistics: bool = False) -> dict:
    """AWQ scale search for one linear layer; returns packed, scales, zeros, s,
    best_alpha (int32 [1] on device), loss (fp64 [n_alpha] on device).  With
    reuse_statistics the statistics of X are taken from `workspace`, which the previous
    call must have filled from the same X (awq_quantize_shared)."""
    _need(W, "W", torch.float16, 2)
    _check_bits(bits)
    _need(X, "X", torch.float16, 2)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or X.device != W.device:
        raise ValueError("X must be fp16 [M][K] on W's device")
    if K % group:
        raise ValueError(f"K={K} is not a multiple of group {group}")
    al = np.ascontiguousarray(default_alpha_grid() if alphas is None else np.asarray(alphas, dtype=np.float32))
    n_alpha = int(al.shape[0])
    if not 1 <= n_alpha <= MAX_ALPHAS:
        raise ValueError(f"need 1..{MAX_ALPHAS} alphas, got {n_alpha}")
    lib = load()
    ws_bytes = int(lib.awq_quantize_workspace_bytes(N, K, M, group, n_alpha))
    if ws_bytes == 0:
        raise ValueError("unsupported sizes for awq_quantize")
    if workspace is None:
        if reuse_statistics:
            raise ValueError("reuse_statistics needs the workspace of the previous call on the same X")
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=W.device)
    elif workspace.numel() * workspace.element_size() < ws_bytes or not workspace.is_cuda:
        raise ValueError(f"workspace must be a GPU buffer of at least {ws_bytes} bytes")
    packed, scales, zeros = empty_packed(N, K, W.device, group, bits)
    s = torch.empty((K,), dtype=torch.float32, device=W.device)
    best = torch.empty((1,), dtype=torch.int32, device=W.device)
    loss = torch.empty((n_alpha,), dtype=torch.float64, device=W.device)
    with torch.cuda.device(W.device):
        check(lib.awq_quantize_shared(W.data_ptr(), X.data_ptr(), N, K, M, group, bits, al.ctypes.data, n_alpha,
                                      int(bool(reuse_statistics)), packed.data_ptr(), scales.data_ptr(),
                                      zeros.data_ptr(), s.data_ptr(), best.data_ptr(), loss.data_ptr(),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(W.device)))
    return dict(packed=packed, scales=scales, zeros=zeros, s=s, best_alpha=best, loss=loss, alphas=al, bits=bits)


# awq_gemm_ws workspaces cached per (device, stream): tile counters start at zero and every
# call leaves them zero; calls on one stream are ordered, so they may share one.
_GEMM_WS = {}


def _gemm_workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _GEMM_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _GEMM_WS[key] = ws
    return ws


def awq_gemm(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
             out: Optional[torch.Tensor] = None, group: int = GROUP, bits: Optional[int] = None,
             workspace="auto") -> torch.Tensor:
    """y = x @ w_hat^T with fp32 accumulation; x fp16 [M][K] (already divided by s).  bits
    (4 or 3) defaults to the width the packed tensor's shape says it was written at.
    workspace: "auto" (awq_gemm_ws with a workspace cached for the device and stream, so the
    GEMM may split its work over the compute units), a zero-initialized uint8 device tensor
    of at least awq_gemm_workspace_bytes(M, N, K, bits) bytes, or None (awq_gemm_bits: whole
    output tiles per block)."""
    _need(x, "x", torch.float16, 2)
    _need(packed, "packed", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    M, K = x.shape
    N = packed.shape[0]
    G = K // group
    if bits is None:
        bits = bits_of(packed, K)
    if packed.shape[1] != packed_words(K, bits) or tuple(scales.shape) != (N, G) or \
            tuple(zeros.shape) != (N, (G + 1) // 2):
        raise ValueError("packed/scales/zeros do not match x's K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be fp16 [M][N]")
    lib = load()
    need = lib.awq_gemm_workspace_bytes(M, N, K, bits) if workspace is not None else 0
    with torch.cuda.device(x.device):
        stream = _stream(x.device)
        if need == 0:
            check(lib.awq_gemm_bits(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                    out.data_ptr(), M, N, K, group, bits, stream))
            return out
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a uint8 device tensor')
            ws = _gemm_workspace(x.device, stream, need)
        else:
            _need(workspace, "workspace", torch.uint8, 1)
            ws = workspace
        check(lib.awq_gemm_ws(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                              out.data_ptr(), M, N, K, group, bits, ws.data_ptr(), ws.numel(), stream))
    return out


def awq_gemm_workspace_bytes(M: int, N: int, K: int, bits: int = 4) -> int:
    """Workspace bytes awq_gemm_ws needs for this product (0: it splits no work)."""
    _check_bits(bits)
    return int(load().awq_gemm_workspace_bytes(int(M), int(N), int(K), int(bits)))


def awq_gemm_kernel(M: int, N: int, K: int, bits: int = 4, group: int = GROUP, workspace: bool = True) -> str:
    """The kernel awq_gemm launches for an M x K input and N x K weights (a host-only dry run of
    its dispatch: the kernel's template arguments, block and grid), with a workspace (as
    awq_gemm's default does) or without."""
    _check_bits(bits)
    buf = ctypes.create_string_buffer(160)
    fn = load().awq_gemm_ws_kernel if workspace else load().awq_gemm_kernel
    check(fn(int(M), int(N), int(K), int(group), int(bits), buf, len(buf)))
    return buf.value.decode()


def awq_scale_input(x: torch.Tensor, s: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """xs = fp16(fp32(x) / s) per input channel (IEEE fp32 division, then fp16); x fp16 [M][K]."""
    _need(x, "x", torch.float16, 2)
    _need(s, "s", torch.float32, 1)
    M, K = x.shape
    if s.shape[0] != K:
        raise ValueError("s must have K entries")
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (M, K):
            raise ValueError("out must be fp16 [M][K]")
    with torch.cuda.device(x.device):
        check(load().awq_scale_input(x.data_ptr(), s.data_ptr(), M, K, out.data_ptr(), _stream(x.device)))
    return out


def awq_gemm_scaled_workspace_bytes(M: int, N: int, K: int, bits: int = 4) -> int:
    return int(load().awq_gemm_scaled_workspace_bytes(M, N, K, bits))


def awq_gemm_scaled(x: torch.Tensor, s: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                    zeros: torch.Tensor, out: Optional[torch.Tensor] = None, group: int = GROUP,
                    bits: Optional[int] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = awq_scale_input(x, s) @ w_hat^T; x fp16 [M][K] not divided by s.  The scaled input
    goes through a workspace of awq_gemm_scaled_workspace_bytes bytes, taken from `workspace`
    or allocated."""
    _need(x, "x", torch.float16, 2)
    _need(s, "s", torch.float32, 1)
    _need(packed, "packed", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    M, K = x.shape
    N = packed.shape[0]
    G = K // group
    if bits is None:
        bits = bits_of(packed, K)
    if s.shape[0] != K or packed.shape[1] != packed_words(K, bits) or tuple(scales.shape) != (N, G) or \
            tuple(zeros.shape) != (N, (G + 1) // 2):
        raise ValueError("s/packed/scales/zeros do not match x's K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be fp16 [M][N]")
    need = awq_gemm_scaled_workspace_bytes(M, N, K, bits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        check(load().awq_gemm_scaled(x.data_ptr(), s.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                                     zeros.data_ptr(), out.data_ptr(), M, N, K, group, bits, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(x.device)))
    return out


ABLATION_ORDER = ("none", "activation", "weight", "random")


def awq_ablation_workspace_bytes(N: int, K: int, M: int, group: int = GROUP) -> int:
    return int(load().awq_ablation_workspace_bytes(N, K, M, group))


def awq_keep_fp16_ablation(W: torch.Tensor, X: torch.Tensor, n_keep: int, random_keep: Optional[torch.Tensor] = None,
                           group: int = GROUP, bits: int = 4, workspace: Optional[torch.Tensor] = None) -> dict:
    """Output MSE of plain rounding with n_keep input channels kept in fp16, chosen by
    activation magnitude, by weight magnitude and at random (random_keep: int32 [n_keep] on
    W's device, the caller's draw); loss fp64 [4] in ABLATION_ORDER."""
    _need(W, "W", torch.float16, 2)
    _need(X, "X", torch.float16, 2)
    _check_bits(bits)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or X.device != W.device:
        raise ValueError("X must be fp16 [M][K] on W's device")
    if not 0 <= n_keep <= K:
        raise ValueError(f"n_keep={n_keep} outside [0, {K}]")
    if n_keep > 0:
        if random_keep is None:
            raise ValueError("random_keep is required when n_keep > 0")
        _need(random_keep, "random_keep", torch.int32, 1)
        if random_keep.shape[0] != n_keep or random_keep.device != W.device:
            raise ValueError("random_keep must be int32 [n_keep] on W's device")
    lib = load()
    ws_bytes = int(lib.awq_ablation_workspace_bytes(N, K, M, group))
    if ws_bytes == 0:
        raise ValueError("unsupported sizes for awq_keep_fp16_ablation")
    if workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=W.device)
    elif workspace.numel() * workspace.element_size() < ws_bytes or not workspace.is_cuda:
        raise ValueError(f"workspace must be a GPU buffer of at least {ws_bytes} bytes")
    keep_act = torch.empty((n_keep,), dtype=torch.int32, device=W.device)
    keep_wt = torch.empty((n_keep,), dtype=torch.int32, device=W.device)
    loss = torch.empty((4,), dtype=torch.float64, device=W.device)
    with torch.cuda.device(W.device):
        check(lib.awq_keep_fp16_ablation(W.data_ptr(), X.data_ptr(), N, K, M, group, bits, n_keep,
                                         _ptr(random_keep) if n_keep > 0 else None, keep_act.data_ptr(),
                                         keep_wt.data_ptr(), loss.data_ptr(), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream(W.device)))
    return dict(loss=loss, keep_activation=keep_act, keep_weight=keep_wt, order=ABLATION_ORDER)


def awq_unpack(packed: torch.Tensor, zeros: torch.Tensor, K: int, group: int = GROUP, bits: Optional[int] = None):
    """Logical codes uint8 [N][K] and zero points uint8 [N][K/g] of a packed layer."""
    _need(packed, "packed", torch.int32, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    if bits is None:
        bits = bits_of(packed, K)
    N = packed.shape[0]
    codes = torch.empty((N, K), dtype=torch.uint8, device=packed.device)
    z = torch.empty((N, K // group), dtype=torch.uint8, device=packed.device)
    with torch.cuda.device(packed.device):
        check(load().awq_unpack_bits(packed.data_ptr(), zeros.data_ptr(), N, K, group, bits, codes.data_ptr(),
                                     z.data_ptr(), _stream(packed.device)))
    return codes, z


__all__ = [n for n in dir() if n.startswith("awq_")] + ["AwqError", "default_alpha_grid", "empty_packed",
                                                        "packed_words", "bits_of", "ABLATION_ORDER"]
