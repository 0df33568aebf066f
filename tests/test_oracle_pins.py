"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one function by a closed form, a brute-force search over a tiny
input, an invariant of the mathematics, or a group worked out by hand.  A
plausible mistake in the oracle (a dropped term, a wrong sign or axis, /16
instead of /15, floor instead of round-half-even, a transposed operand) fails
at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from gen import activations_fp16, normal_fp16


def F(x):
    return Fraction(float(x))


# ----------------------------------------------------------------- channel stats
def test_mean_abs_equals_exact_sum_over_rows():
    g = np.random.default_rng(1)
    # fp16 values spanning subnormals to large magnitudes, both signs
    mag = np.exp2(g.integers(-24, 15, size=(37, 16))).astype(np.float64)
    X = (g.choice([-1.0, 1.0], size=mag.shape) * mag * g.uniform(1, 2, size=mag.shape)).astype(np.float16)
    a = O.channel_mean_abs(X)
    for k in range(X.shape[1]):
        exact = math.fsum(abs(float(v)) for v in X[:, k])  # correctly rounded sum
        assert a[k] == exact / X.shape[0]


def test_mean_abs_constant_magnitude_and_signs():
    M, K = 64, 8
    g = np.random.default_rng(2)
    c = np.array([0.0, 2.0 ** -24, 0.5, 1.0, 3.0, 4.0, 1000.0, 65504.0])
    X = (g.choice([-1.0, 1.0], size=(M, K)) * c[None, :]).astype(np.float16)
    assert np.array_equal(O.channel_mean_abs(X), c)


# ----------------------------------------------------------------- s(alpha)
def test_scales_closed_forms():
    a = np.array([0.0, 1.0, 4.0, 16.0, 0.25, 2.0 ** 20, 3.0])
    assert np.array_equal(O.scales_for_alpha(a, 0.0), np.ones(7, np.float32))
    s = O.scales_for_alpha(a, 0.5)
    assert s[0] == 1.0                      # a = 0 -> s = 1
    assert list(s[1:6]) == [1.0, 2.0, 4.0, 0.5, 1024.0]
    assert s[6] == np.float32(math.sqrt(3.0))
    s25 = O.scales_for_alpha(np.array([16.0, 2.0 ** -8]), 0.25)
    assert list(s25) == [2.0, 0.25]


def test_scales_monotone_in_magnitude():
    a = np.sort(np.random.default_rng(3).uniform(1e-3, 1e3, 500))
    for al in (0.05, 0.5, 0.95):
        s = O.scales_for_alpha(a, al)
        assert np.all(np.diff(s) >= 0)
        assert np.all(np.abs(s.astype(np.float64) - a ** np.float64(np.float32(al))) <= 2.0 ** -24 * s)


def test_alpha_grid():
    g = O.alpha_grid(20)
    assert len(g) == 20 and g[0] == 0.0 and g[10] == 0.5 and g[19] < 1.0
    assert np.all(np.diff(g) > 0)


# ----------------------------------------------------------------- quantizer
def _hand_group(values, fill):
    v = np.full(128, fill, dtype=np.float32)
    v[: len(values)] = np.array(values, dtype=np.float32)
    return v[None, :]


def test_quantizer_hand_worked_mixed_sign_group():
    # lo = -1.5, hi = 6.0: step = 7.5 / 15 = 0.5 exactly, fp16 keeps it; z = rint(1.5 / 0.5) = 3.
    # q = rint(2 v) + 3, with halves going to the even neighbour:
    #  -1.5 -> -3 -> 0      6.0 -> 12 -> 15     0.25 -> 0.5 -> 0 -> 3    0.75 -> 1.5 -> 2 -> 5
    #  1.25 -> 2.5 -> 2 -> 5   -0.25 -> -0.5 -> 0 -> 3   -0.75 -> -1.5 -> -2 -> 1
    #  5.9 -> 11.8 -> 12 -> 15   0.0 -> 3   fill 1.0 -> 2 -> 5
    V = _hand_group([-1.5, 6.0, 0.25, 0.75, 1.25, -0.25, -0.75, 5.9, 0.0], 1.0)
    q, z, sc = O.quantize_groups(V)
    assert sc[0, 0] == np.float16(0.5) and z[0, 0] == 3
    assert list(q[0, :9]) == [0, 15, 3, 5, 5, 3, 1, 15, 3]
    assert np.all(q[0, 9:] == 5)


def test_quantizer_hand_worked_three_bit_group():
    # 3-bit codes (0..7): lo = -1.5, hi = 2.0, step = 3.5 / 7 = 0.5 exactly; z = rint(1.5 / 0.5) = 3.
    # q = rint(2 v) + 3 clamped to [0, 7], halves to the even neighbour:
    #  -1.5 -> 0    2.0 -> 4 + 3 = 7    0.25 -> 0 -> 3    0.75 -> 2 -> 5    1.25 -> 2 -> 5
    #  -0.75 -> -2 -> 1    1.9 -> 3.8 -> 4 -> 7    0.0 -> 3    fill 1.0 -> 2 -> 5
    V = _hand_group([-1.5, 2.0, 0.25, 0.75, 1.25, -0.75, 1.9, 0.0], 1.0)
    q, z, sc = O.quantize_groups(V, bits=3)
    assert sc[0, 0] == np.float16(0.5) and z[0, 0] == 3
    assert list(q[0, :8]) == [0, 7, 3, 5, 5, 1, 7, 3]
    assert np.all(q[0, 8:] == 5)
    # the same values at 4 bits: step 3.5 / 15 rounds to an fp16 that is not 0.5
    q4, z4, sc4 = O.quantize_groups(V, bits=4)
    assert sc4[0, 0] != sc[0, 0] and q4.max() > 7


def test_quantizer_hand_worked_positive_group_fp16_step():
    # lo = min(0, 1) = 0, hi = 3: step = fp32(0.2); the nearest fp16 is 1638 * 2**-13
    # = 0.199951171875 (0.2 / 2**-13 = 1638.4).  z = 0.  q = rint(v / 0.19995...):
    # 1 -> 5.0012 -> 5, 2 -> 10.0024 -> 10, 3 -> 15.0037 -> 15, 2.9 -> 14.5035 -> 15.
    V = _hand_group([1.0, 2.0, 3.0, 2.9], 1.0)
    q, z, sc = O.quantize_groups(V)
    assert float(sc[0, 0]) == 1638 * 2.0 ** -13 and z[0, 0] == 0
    assert list(q[0, :4]) == [5, 10, 15, 15]


def _fp16_rne_bits(u32):
    """fp32 bit patterns -> fp16 bit patterns, round to nearest even, by integer arithmetic
    alone (finite inputs; overflow to inf).  Independent of numpy's cast, which the oracle
    uses for the fp16 group step."""
    u = np.asarray(u32, dtype=np.uint64)
    sign = (u >> np.uint64(31)) << np.uint64(15)
    exp = ((u >> np.uint64(23)) & np.uint64(0xFF)).astype(np.int64)
    man = (u & np.uint64(0x7FFFFF)) | np.uint64(0x800000)      # 24-bit significand with the hidden bit
    out = np.zeros(u.shape, dtype=np.uint64)
    e16 = exp - 127 + 15                                         # fp16 biased exponent if normal
    # number of significand bits to drop: 13 for normals, more for subnormals (value = m * 2^(e-24) ...)
    shift = np.where(e16 >= 1, 13, 13 + 1 - e16).astype(np.int64)
    shift = np.minimum(shift, 40)
    sh = shift.astype(np.uint64)
    q = man >> sh
    rem = man - (q << sh)
    half = np.uint64(1) << (sh - np.uint64(1))
    up = (rem > half) | ((rem == half) & ((q & np.uint64(1)) == np.uint64(1)))
    q = q + up.astype(np.uint64)
    # q is the fp16 significand (with hidden bit for normals); re-assemble (a carry bumps the exponent)
    normal = e16 >= 1
    eo = np.where(normal, e16, 0).astype(np.int64)
    carry = normal & (q >= np.uint64(0x800))
    q = np.where(carry, q >> np.uint64(1), q)
    eo = np.where(carry, eo + 1, eo)
    bits = np.where(normal, (eo.astype(np.uint64) << np.uint64(10)) | (q & np.uint64(0x3FF)), q)
    bits = np.where(normal & (eo >= 31), np.uint64(0x7C00), bits)  # overflow -> inf
    zero = exp == 0                                              # fp32 zero or subnormal -> +-0 in fp16
    bits = np.where(zero, np.uint64(0), bits)
    return (sign | bits).astype(np.uint16)


def test_fp16_rounding_is_round_to_nearest_even():
    # The oracle rounds the group step to fp16 with numpy's cast: pin that cast against an
    # integer-only round-to-nearest-even on 2^20 random patterns spanning normals, fp16
    # subnormals, overflow and exact ties.
    g = np.random.default_rng(55)
    u = g.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    e = g.integers(127 - 30, 127 + 17, size=u.shape[0]).astype(np.uint32)   # exponents around the fp16 range
    u = (u & np.uint32(0x807FFFFF)) | (e << np.uint32(23))
    ties = (u[: 1 << 16] & np.uint32(0xFFFFE000)) | np.uint32(0x1000)        # exactly half an fp16 ulp
    u = np.concatenate([u, ties])
    want = _fp16_rne_bits(u)
    with np.errstate(over="ignore"):
        got = u.view(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    # hand cases: 1 + 2^-11 ties down to 1; 1 + 3 * 2^-11 ties up to 1 + 2^-9; 65520 overflows
    with np.errstate(over="ignore"):
        for v, r in [(1 + 2.0 ** -11, 1.0), (1 + 3 * 2.0 ** -11, 1 + 2.0 ** -9), (65520.0, np.inf), (2.0 ** -25, 0.0)]:
            assert float(np.float32(v).astype(np.float16)) == r


def test_quantizer_hand_worked_negative_and_zero_groups():
    # all-negative: lo = -3, hi = 0, same step 0.19995...; z = rint(15.0037) = 15;
    # -3 -> rint(-15.0037) + 15 = 0, -1.5 -> rint(-7.5018) + 15 = -8 + 15 = 7.
    V = _hand_group([-3.0, -1.5], -3.0)
    q, z, sc = O.quantize_groups(V)
    assert z[0, 0] == 15 and list(q[0, :2]) == [0, 7]
    # all-zero group: the step floors at 2**-14 (smallest normal fp16), z = 0, q = 0
    q, z, sc = O.quantize_groups(np.zeros((1, 128), np.float32))
    assert float(sc[0, 0]) == 2.0 ** -14 and z[0, 0] == 0 and np.all(q == 0)


def _fp16_neighbours(x16):
    up = np.nextafter(x16, np.float16(np.inf))
    dn = np.nextafter(x16, np.float16(-np.inf))
    return dn, up


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("group", [8, 16, 128])
def test_quantizer_brute_force_nearest(group, bits):
    qmax = 2 ** bits - 1
    g = np.random.default_rng(10 + group + bits)
    N, K = 6, group * 3
    V = (g.standard_normal((N, K)) * g.choice([0.01, 1.0, 50.0], size=(N, 1))).astype(np.float32)
    V[0, :group] = np.abs(V[0, :group])            # a one-signed group
    V[1, group:2 * group] = -np.abs(V[1, group:2 * group])
    q, z, sc16 = O.quantize_groups(V, group, bits)
    assert q.max() <= qmax and z.max() <= qmax
    for n in range(N):
        for j in range(K // group):
            vs = V[n, j * group:(j + 1) * group]
            lo = min(0.0, float(vs.min()))
            hi = max(0.0, float(vs.max()))
            step = max(F(np.float32(np.float32(hi) - np.float32(lo))) / qmax, F(2.0 ** -14))
            sc = F(sc16[n, j])
            # sc is the fp16 nearest to the float32 step (ties to even mantissa)
            dn, up = _fp16_neighbours(sc16[n, j])
            d0 = abs(sc - step)
            assert d0 <= abs(F(dn) - step) and d0 <= abs(F(up) - step)
            # z is the nearest integer in [0, qmax] to -lo / sc (slack: one fp32 rounding)
            t = F(-lo) / sc
            dz = [abs(t - c) for c in range(qmax + 1)]
            assert dz[z[n, j]] <= min(dz) + Fraction(1, 2 ** 19)
            # every code is a nearest grid point (q - z) * sc over q in [0, qmax]
            for i, v in enumerate(vs):
                d = [abs(F(v) - (c - int(z[n, j])) * sc) for c in range(qmax + 1)]
                assert d[q[n, j * group + i]] <= min(d) + sc / 2 ** 19


@pytest.mark.parametrize("bits", [3, 4])
def test_quantizer_error_bound_and_ranges(bits):
    qmax = 2 ** bits - 1
    W = normal_fp16((64, 1024), 0.02, seed=11)
    a = O.channel_mean_abs(activations_fp16(64, 1024, seed=12))
    for al in (0.0, 0.35, 0.9):
        q, z, sc16, s = O.quantize_at(W, a, al, bits=bits)
        V = O.scale_weights(W, s).astype(np.float64)
        assert q.max() <= qmax and z.max() <= qmax
        assert np.all(np.isfinite(sc16.astype(np.float32))) and np.all(sc16 > 0)
        Wh = O.dequantize(q, z, sc16)
        scf = np.repeat(sc16.astype(np.float64), 128, axis=1)
        zz = np.repeat(z.astype(np.float64), 128, axis=1)
        unclamped = (np.rint(V / scf) + zz >= 0) & (np.rint(V / scf) + zz <= qmax)
        err = np.abs(V - Wh)
        assert np.all(err[unclamped] <= scf[unclamped] * (0.5 + 2.0 ** -20))
        # clamped elements can only exist because fp16 rounding shrank the step
        assert np.all(err <= scf * (0.5 + (qmax + 1) * 2.0 ** -11))


def test_quantizer_power_of_two_covariance():
    V = (np.random.default_rng(13).standard_normal((8, 512)) * 0.3).astype(np.float32)
    q0, z0, s0 = O.quantize_groups(V)
    for e in (-3, 2, 5):
        q1, z1, s1 = O.quantize_groups(V * np.float32(2.0 ** e))
        assert np.array_equal(q0, q1) and np.array_equal(z0, z1)
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** e)


# ----------------------------------------------------------------- a lossless construction
def _on_grid_layer(N=8, K=256, M=16, seed=20):
    """W and X for which quantization at alpha = 0.5 is exact.

    |X[:, k]| = 4**e_k (random signs) so a_k = 4**e_k and s_k(0.5) = 2**e_k exactly.
    Per group the scaled weights V = (c - z0) * 2**-6 with codes c in [0, 15] that hit
    both 0 and 15, and 0 <= z0 <= 15: the range is exactly 15 * 2**-6 and contains 0, so
    the quantizer must return step 2**-6, zero z0 and codes c.  W = V / s is exact fp16.
    """
    g = np.random.default_rng(seed)
    e = g.integers(-1, 2, size=K)
    X = (g.choice([-1.0, 1.0], size=(M, K)) * (4.0 ** e)[None, :]).astype(np.float16)
    c = g.integers(0, 16, size=(N, K))
    c[:, 0::128] = 0
    c[:, 1::128] = 15
    z0 = g.integers(0, 16, size=(N, K // 128))
    V = (c - np.repeat(z0, 128, axis=1)) * 2.0 ** -6
    W = (V / 2.0 ** e[None, :]).astype(np.float16)
    assert np.array_equal(W.astype(np.float64) * 2.0 ** e[None, :], V)
    return W, X, c, z0


def test_lossless_construction_three_bit():
    """Codes in [0, 7] hitting both ends of every group, step 2**-5: exact at 3 bits."""
    g = np.random.default_rng(21)
    N, K = 8, 256
    c = g.integers(0, 8, size=(N, K))
    c[:, 0::128] = 0
    c[:, 1::128] = 7
    z0 = g.integers(0, 8, size=(N, K // 128))
    W = ((c - np.repeat(z0, 128, axis=1)) * 2.0 ** -5).astype(np.float16)
    q, z, sc16 = O.quantize_groups(W.astype(np.float32), bits=3)
    assert np.array_equal(q, c) and np.array_equal(z, z0) and np.all(sc16 == np.float16(2.0 ** -5))
    assert np.array_equal(O.dequantize(q, z, sc16), W.astype(np.float64))


def test_lossless_construction_dequantizes_exactly():
    W, X, c, z0 = _on_grid_layer()
    a = O.channel_mean_abs(X)
    q, z, sc16, s = O.quantize_at(W, a, 0.5)
    assert np.array_equal(q, c) and np.array_equal(z, z0) and np.all(sc16 == np.float16(2.0 ** -6))
    assert np.array_equal(O.effective_weight(q, z, sc16, s), W.astype(np.float64))
    assert O.output_mse(X, O.weight_error(W, q, z, sc16, s)) == 0.0


def test_search_known_answer():
    W, X, _, _ = _on_grid_layer()
    r = O.search(W, X)
    assert r["alpha_index"] == 10 and r["losses"][10] == 0.0
    assert np.all(np.delete(r["losses"], 10) > 0)


def test_scaling_invariance_fp64():
    # (W diag(s)) (diag(1/s) x) = W x: the effective weight divides by s along the input axis.
    g = np.random.default_rng(21)
    W = normal_fp16((32, 512), 0.02, seed=22)
    s = g.uniform(0.1, 30.0, 512).astype(np.float32)
    q, z, sc16 = O.quantize_groups(O.scale_weights(W, s))
    x = g.standard_normal((5, 512))
    y1 = x @ O.effective_weight(q, z, sc16, s).T
    y2 = (x / s.astype(np.float64)[None, :]) @ O.dequantize(q, z, sc16).T
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y1))
    Wl, Xl, _, _ = _on_grid_layer()
    ql, zl, scl, sl = O.quantize_at(Wl, O.channel_mean_abs(Xl), 0.5)
    xl = g.standard_normal((3, Wl.shape[1]))
    assert np.max(np.abs(xl @ O.effective_weight(ql, zl, scl, sl).T - xl @ Wl.astype(np.float64).T)) <= \
        1e-12 * np.max(np.abs(xl @ Wl.astype(np.float64).T))


def test_scaled_input_special_cases():
    # s = 1 leaves x unchanged; s = 2^e is an exact exponent shift (no value here underflows)
    x = activations_fp16(6, 256, seed=31)
    assert np.array_equal(O.scaled_input(x, np.ones(256, np.float32)).view(np.uint16), x.view(np.uint16))
    e = np.random.default_rng(32).integers(-6, 7, 256)
    s = np.ldexp(np.ones(256, np.float32), e).astype(np.float32)
    assert np.array_equal(O.scaled_input(x, s), np.ldexp(x.astype(np.float64), -e[None, :]).astype(np.float16))
    # one rounding: every value is the fp16 nearest to the exact quotient, or ties to it within half an fp16 ulp
    s = np.random.default_rng(33).uniform(0.2, 9.0, 256).astype(np.float32)
    xs = O.scaled_input(x, s).astype(np.float64)
    exact = x.astype(np.float64) / s.astype(np.float64)[None, :]
    ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(xs - exact) <= 0.5 * ulp * (1 + 2.0 ** -20))
    for i, j in [(0, 0), (3, 17), (5, 255)]:  # brute force: the nearer of the two fp16 neighbours
        q = Fraction(float(x[i, j])) / Fraction(float(s[j]))
        lo = np.float16(float(q))
        cands = {float(lo), float(np.nextafter(lo, np.float16(np.inf))), float(np.nextafter(lo, np.float16(-np.inf)))}
        best = min(abs(Fraction(c) - q) for c in cands)
        assert abs(Fraction(float(O.scaled_input(x, s)[i, j])) - q) == best


def test_scaled_input_product_matches_unscaled_layer():
    # (x / s) w_hat^T = x (w_hat / s)^T up to the fp16 rounding of x / s, whose effect is
    # bounded by sum_k |x_k / s_k| 2^-11 |w_hat_nk|.
    W = normal_fp16((48, 512), 0.02, seed=34)
    X = activations_fp16(64, 512, seed=35)
    q, z, sc16, s = O.quantize_at(W, O.channel_mean_abs(X), 0.5)
    x = activations_fp16(4, 512, seed=36)
    y = O.gemm(O.scaled_input(x, s), q, z, sc16)
    ref = x.astype(np.float64) @ O.effective_weight(q, z, sc16, s).T
    bound = (np.abs(x.astype(np.float64) / s.astype(np.float64)[None, :]) * 2.0 ** -11) @ np.abs(O.dequantize(q, z, sc16)).T
    assert np.all(np.abs(y - ref) <= bound * (1 + 1e-9)) and np.max(np.abs(y - ref)) > 0


# ----------------------------------------------------------------- loss
def test_loss_brute_force_loops():
    g = np.random.default_rng(30)
    M, K, N = 3, 8, 2
    X = g.standard_normal((M, K)).astype(np.float16)
    E = g.standard_normal((N, K)) * 1e-3
    ref = math.fsum(math.fsum(float(X[t, k]) * E[n, k] for k in range(K)) ** 2
                    for t in range(M) for n in range(N)) / (M * N)
    assert abs(O.output_mse(X, E) - ref) <= 1e-12 * ref


def test_loss_gram_identity():
    X = activations_fp16(300, 256, seed=31)
    E = np.random.default_rng(32).standard_normal((40, 256)) * 1e-3
    d = O.output_mse(X, E)
    gm = O.output_mse_gram(O.gram(X), E, 300)
    assert abs(d - gm) <= 1e-10 * d


# ----------------------------------------------------------------- search
def test_alpha_zero_is_round_to_nearest():
    W = normal_fp16((64, 512), 0.02, seed=40)
    X = activations_fp16(64, 512, seed=41)
    q0, z0, sc0, s0 = O.quantize_at(W, O.channel_mean_abs(X), 0.0)
    qr, zr, scr = O.quantize_groups(W.astype(np.float32))
    assert np.all(s0 == 1.0)
    assert np.array_equal(q0, qr) and np.array_equal(z0, zr) and np.array_equal(sc0, scr)
    r = O.search(W, X)
    assert r["losses"][0] == O.output_mse(X, O.weight_error(W, qr, zr, scr, s0))


def test_search_never_worse_than_round_to_nearest():
    W = normal_fp16((512, 512), 0.02, seed=1001)
    X = activations_fp16(64, 512, seed=1002)
    r = O.search(W, X)
    assert r["losses"][r["alpha_index"]] <= r["losses"][0]
    assert r["losses"][r["alpha_index"]] == r["losses"].min()
    assert r["alpha_index"] == int(np.argmin(r["losses"]))


def test_search_forced_tie_power_of_two():
    # |x| = 4 everywhere -> a = 4, s(alpha_10 = 0.5) = 2: scaling by 2 is exact, so the codes
    # and the loss at alpha_10 equal those at alpha_0 exactly.
    g = np.random.default_rng(50)
    X = (g.choice([-4.0, 4.0], size=(32, 256))).astype(np.float16)
    W = normal_fp16((16, 256), 0.02, seed=51)
    r = O.search(W, X)
    assert r["losses"][10] == r["losses"][0]
    a = O.channel_mean_abs(X)
    qa, za, _, _ = O.quantize_at(W, a, 0.0)
    qb, zb, _, _ = O.quantize_at(W, a, 0.5)
    assert np.array_equal(qa, qb) and np.array_equal(za, zb)
    assert r["alpha_index"] != 10  # the first of the tied pair wins, or a strictly better alpha


# ----------------------------------------------------------------- product
def test_gemm_brute_force_loops():
    g = np.random.default_rng(60)
    N, K, M = 3, 256, 2
    q = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = g.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    sc = g.uniform(1e-3, 1e-1, size=(N, K // 128)).astype(np.float16)
    x = g.standard_normal((M, K)).astype(np.float16)
    y = O.gemm(x, q, z, sc)
    for m in range(M):
        for n in range(N):
            ref = math.fsum(float(x[m, k]) * (int(q[n, k]) - int(z[n, k // 128])) * float(sc[n, k // 128])
                            for k in range(K))
            assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_gemm_one_hot_and_zero_codes():
    g = np.random.default_rng(61)
    N, K = 4, 384
    q = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = g.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    sc = g.uniform(1e-3, 1e-1, size=(N, K // 128)).astype(np.float16)
    for k in (0, 1, 127, 128, 200, 383):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        y = O.gemm(x, q, z, sc)[0]
        for n in range(N):
            assert y[n] == (int(q[n, k]) - int(z[n, k // 128])) * float(sc[n, k // 128])
    qz = np.repeat(z, 128, axis=1)
    assert np.all(O.gemm(g.standard_normal((2, K)).astype(np.float16), qz, z, sc) == 0.0)


# ----------------------------------------------------------------- keep-fp16 ablation
def test_top_channels_hand_ranking():
    v = np.array([1.0, 3.0, 3.0, 2.0, 5.0, 0.0, 3.0])
    assert list(O.top_channels(v, 4)) == [4, 1, 2, 6]  # 5, then the three 3s by index
    assert list(O.top_channels(v, 0)) == []
    assert sorted(O.top_channels(v, 7)) == list(range(7))


def test_keep_fp16_extremes():
    W = normal_fp16((16, 256), 0.02, seed=30)
    X = activations_fp16(24, 256, seed=31)
    r = O.keep_fp16_ablation(W, X, 256, np.arange(256))
    assert np.all(r["losses"][1:] == 0.0)  # every channel kept: nothing is rounded
    r0 = O.keep_fp16_ablation(W, X, 0, np.zeros(0, np.int32))
    L0 = O.search(W, X, alphas=np.zeros(1, np.float32))["losses"][0]
    assert np.all(r0["losses"] == L0) and L0 > 0  # nothing kept: plain rounding


def test_keep_fp16_loss_brute_force_loops():
    W = normal_fp16((4, 128), 0.05, seed=32)
    X = activations_fp16(5, 128, seed=33)
    keep = np.array([3, 70], np.int32)
    q, z, sc = O.quantize_groups(W.astype(np.float32))
    L = 0.0
    for t in range(5):
        for n in range(4):
            acc = 0.0
            for k in range(128):
                if k in (3, 70):
                    continue
                w_hat = (int(q[n, k]) - int(z[n, 0])) * float(sc[n, 0])
                acc += float(X[t, k]) * (w_hat - float(W[n, k]))
            L += acc * acc
    L /= 20.0
    r = O.keep_fp16_ablation(W, X, 2, keep)
    assert abs(r["losses"][3] - L) <= 1e-12 * L


def test_keep_fp16_gram_equals_direct():
    W = normal_fp16((32, 256), 0.02, seed=34)
    X = activations_fp16(300, 256, seed=35, lognormal=True)
    rnd = np.random.default_rng(36).permutation(256)[:3].astype(np.int32)
    d = O.keep_fp16_ablation(W, X, 3, rnd, use_gram=False)["losses"]
    g = O.keep_fp16_ablation(W, X, 3, rnd, use_gram=True)["losses"]
    assert np.all(np.abs(d - g) <= 1e-10 * d)


def test_keep_fp16_activation_channels_are_the_outliers():
    """With a few input channels scaled x20 (the synthetic salient channels), keeping the
    channels of largest mean |x| keeps exactly those, and removes their error terms."""
    K = 512
    W = normal_fp16((64, K), 0.02, seed=37)
    X = activations_fp16(256, K, seed=38)  # 1% of channels (5) carry x20 outliers
    a = O.channel_mean_abs(X)
    outliers = np.sort(np.argsort(-a)[:5])
    assert np.all(a[outliers] > 10 * np.median(a))
    r = O.keep_fp16_ablation(W, X, 5, np.arange(5, dtype=np.int32))
    assert np.array_equal(np.sort(r["keep_activation"]), outliers)
    assert r["losses"][1] < r["losses"][0]
