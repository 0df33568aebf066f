"""Host-side reader and writer of the packed 4-bit and 3-bit formats, written from
their description in include/awq.h (independent of the library's own unpack kernels).

  packed  uint32 [N][K/8]: the code of channel 8w+i sits in nibble 4*(i%2) + i//2 of word w
  zeros   uint8 [N][ceil(G/2)]: group j in byte j//2, low nibble for even j
"""
import numpy as np

GROUP = 128


def nibble(i: int) -> int:
    return 4 * (i % 2) + i // 2


def decode_codes(packed: np.ndarray, K: int) -> np.ndarray:
    words = np.ascontiguousarray(packed).view(np.uint32).reshape(packed.shape[0], K // 8)
    codes = np.empty((words.shape[0], K // 8, 8), dtype=np.uint8)
    for i in range(8):
        codes[:, :, i] = (words >> np.uint32(4 * nibble(i))) & np.uint32(15)
    return codes.reshape(words.shape[0], K)


def decode_zeros(zeros: np.ndarray, G: int) -> np.ndarray:
    z = np.empty((zeros.shape[0], G), dtype=np.uint8)
    for j in range(G):
        z[:, j] = (zeros[:, j // 2] >> (4 * (j % 2))) & 15
    return z


def encode(codes: np.ndarray, zeros: np.ndarray):
    """(codes uint8 [N][K], zeros uint8 [N][G]) -> (packed int32 [N][K/8], zeros bytes [N][ceil(G/2)])."""
    N, K = codes.shape
    G = zeros.shape[1]
    c = codes.reshape(N, K // 8, 8).astype(np.uint32)
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for i in range(8):
        words |= c[:, :, i] << np.uint32(4 * nibble(i))
    zb = np.zeros((N, (G + 1) // 2), dtype=np.uint8)
    for j in range(G):
        zb[:, j // 2] |= (zeros[:, j].astype(np.uint8) & 15) << (4 * (j % 2))
    return words.view(np.int32), zb


# 3-bit format: per 32 channels of a row, three words; channel pair p = 0..14 (channels
# 2p, 2p+1) in word p // 5, fields at bits 3 (p % 5) and 16 + 3 (p % 5); bit b of the
# codes of channels 30 and 31 in bits 15 and 31 of word b.
def _field3(ch: int):
    """(word, bit offset) of the 3-bit field of chunk channel ch < 30."""
    p = ch // 2
    return p // 5, 3 * (p % 5) + 16 * (ch % 2)


def encode3(codes: np.ndarray, zeros: np.ndarray):
    """(codes uint8 [N][K] in 0..7, zeros uint8 [N][G]) -> (packed int32 [N][3K/32], zeros bytes)."""
    N, K = codes.shape
    c = codes.reshape(N, K // 32, 32).astype(np.uint32)
    words = np.zeros((N, K // 32, 3), dtype=np.uint32)
    for ch in range(30):
        t, off = _field3(ch)
        words[:, :, t] |= (c[:, :, ch] & np.uint32(7)) << np.uint32(off)
    for b in range(3):
        words[:, :, b] |= ((c[:, :, 30] >> np.uint32(b)) & np.uint32(1)) << np.uint32(15)
        words[:, :, b] |= ((c[:, :, 31] >> np.uint32(b)) & np.uint32(1)) << np.uint32(31)
    _, zb = encode(np.zeros((N, K), np.uint8), zeros)
    return words.reshape(N, 3 * (K // 32)).view(np.int32), zb


def decode_codes3(packed: np.ndarray, K: int) -> np.ndarray:
    N = packed.shape[0]
    w = np.ascontiguousarray(packed).view(np.uint32).reshape(N, K // 32, 3)
    codes = np.empty((N, K // 32, 32), dtype=np.uint8)
    for ch in range(30):
        t, off = _field3(ch)
        codes[:, :, ch] = (w[:, :, t] >> np.uint32(off)) & np.uint32(7)
    for ch, at in ((30, 15), (31, 31)):
        v = np.zeros((N, K // 32), dtype=np.uint32)
        for b in range(3):
            v |= ((w[:, :, b] >> np.uint32(at)) & np.uint32(1)) << np.uint32(b)
        codes[:, :, ch] = v
    return codes.reshape(N, K)


def rel_fro(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y))


def assert_y_close(y: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """Tolerance for fp16 outputs of the W4A16 product: relative Frobenius error <= 1e-3 and
    max |dy| <= 1e-2 * max |y_ref|."""
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), what
    rf = rel_fro(y, ref)
    mx = float(np.max(np.abs(y - ref))) if y.size else 0.0
    lim = 1e-2 * float(np.max(np.abs(ref))) if y.size else 0.0
    assert rf <= 1e-3, f"{what}: rel Frobenius {rf:.3e} > 1e-3"
    assert mx <= lim or mx == 0.0, f"{what}: max |dy| {mx:.3e} > {lim:.3e}"
