"""The division the fused decode GEMV performs on its x load, checked on the CPU.

The kernel divides x by s without a division instruction, with inv = RN(1/s):
q0 = RN(x * inv); q1 = RN(q0 + RN(x - s q0) * inv) (two fmas), which is within one ulp of x / s;
r = x - s q1 (exact, one fma); q = RN(q1 + r * inv) (one fma); q0 is kept when it is 0.  By
Markstein's theorem on division with a correctly rounded reciprocal the last step gives the
correctly rounded fp32 quotient once q1 is faithful, while x / s is a normal number, which the
library's contract guarantees by asking for s in [2^-64, 2^64] (fp16 x lies in [2^-24, 65504]).
One step from q0 alone is not enough: q0 can be 1.1 ulp off, and then x - s q0 is not exact.
Here the same steps are carried out exactly in fp64 and compared with numpy's IEEE fp32 division
over every finite fp16 x and a spread of s, then rounded to fp16 as the kernel does.  (Not an
oracle test: the oracle divides.)
"""
import numpy as np
import pytest


def _all_finite_fp16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    return x[np.isfinite(x)]


def _round_exact_sum_to_f32(a, b):
    """RN32(a + b) for float64 arrays a, b whose exact sum may need more than 53 bits: the
    float64 sum u and its exact error e (TwoSum) decide the fp32 rounding; only when u is
    exactly halfway between two fp32 values does e break the tie."""
    u = a + b
    bv = u - a
    e = (a - (u - bv)) + (b - bv)
    v = u.astype(np.float32)
    lo = np.nextafter(v, np.float32(-np.inf))
    hi = np.nextafter(v, np.float32(np.inf))
    mid_lo = (v.astype(np.float64) + lo.astype(np.float64)) / 2
    mid_hi = (v.astype(np.float64) + hi.astype(np.float64)) / 2
    # u sits on a midpoint and was rounded to v: move to the neighbour on e's side if needed
    v = np.where((u == mid_hi) & (e > 0), hi, v)
    v = np.where((u == mid_lo) & (e < 0), lo, v)
    return v


def _residual_step(q, x32, s, inv, exact):
    """RN(q + RN(x - s q) inv): x - s q is exact in fp64 (s q has 48 bits, x lies within its
    span), rounded once to fp32 as the fma rounds it; then the second fma's exact sum."""
    r = x32.astype(np.float64) - s.astype(np.float64) * q.astype(np.float64)
    r32 = r.astype(np.float32)
    if exact:
        assert np.array_equal(r32.astype(np.float64), r), "the residual is exact in fp32"
    t = r32.astype(np.float64) * inv.astype(np.float64)        # exact product (48 bits)
    return _round_exact_sum_to_f32(q.astype(np.float64), t)


def _markstein(x32, s):
    inv = np.float32(1.0) / s                                  # correctly rounded reciprocal
    q0 = (x32 * inv).astype(np.float32)                        # RN(x inv)
    q1 = _residual_step(q0, x32, s, inv, exact=False)
    exact_q = np.abs(q1.astype(np.float64) - x32.astype(np.float64) / s.astype(np.float64))
    assert np.all(exact_q <= np.spacing(np.abs(q1)).astype(np.float64)), "q1 is faithful"
    q2 = _residual_step(q1, x32, s, inv, exact=True)
    return np.where(q0 == 0, q0, q2)


def test_one_step_is_not_enough():
    """The case that makes the first step necessary: q0 is 1.1 ulp from x / s."""
    s = np.float32(9.845766e-20)
    x = np.float32(np.float16(5.3346157e-05))
    inv = np.float32(1.0) / s
    q0 = np.float32(x * inv)
    r = np.float64(x) - np.float64(s) * np.float64(q0)
    assert np.float64(np.float32(r)) != r                     # x - s q0 is not exact in fp32
    assert _markstein(np.array([x]), np.array([s]))[0] == x / s


def _s_values():
    g = np.random.default_rng(20260)
    mant = np.concatenate([
        np.array([1.0, 1.0 + 2.0 ** -23, 2.0 - 2.0 ** -23, 1.5, 1.25, 1.75, 1.0 + 2.0 ** -12, 1.999]),
        1.0 + g.random(72)])
    expo = np.concatenate([np.array([-64, -45, -20, -1, 0, 1, 15, 16, 40, 64]), g.integers(-64, 64, 10)])
    s = (mant[:, None] * np.exp2(expo[None, :].astype(np.float64))).reshape(-1).astype(np.float32)
    s = s[(s >= np.float32(2.0 ** -64)) & (s <= np.float32(2.0 ** 64))]
    return np.unique(np.concatenate([s, np.float32([65504.0, 2.0 ** -45])]))


@pytest.mark.parametrize("chunk", range(4))
def test_residual_step_is_the_correctly_rounded_quotient(chunk):
    x = _all_finite_fp16().astype(np.float32)
    svals = np.array_split(_s_values(), 4)[chunk]
    for s0 in svals:
        s = np.full(x.shape, s0, np.float32)
        want = x / s                                           # numpy: IEEE fp32 division
        got = _markstein(x, s)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"s={s0!r}"
        # and the fp16 value the kernel feeds to the products (overflow to inf on both sides)
        with np.errstate(over="ignore"):
            assert np.array_equal(got.astype(np.float16).view(np.uint16), want.astype(np.float16).view(np.uint16))


def test_tie_breaking_helper():
    """The exact-sum rounding above on hand-made halfway cases."""
    one = np.float64(1.0)
    half_ulp = 2.0 ** -24
    a = np.array([one, one, one])
    b = np.array([half_ulp, half_ulp + 2.0 ** -60, half_ulp - 2.0 ** -60])
    got = _round_exact_sum_to_f32(a, b)
    assert got[0] == np.float32(1.0)                           # tie to even
    assert got[1] == np.nextafter(np.float32(1.0), np.float32(2.0))
    assert got[2] == np.float32(1.0)
