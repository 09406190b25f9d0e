"""The Q8_1 kernel forms 127 / m (m in [0.5, 1), the block's amax scaled by
a power of two) as: r = rcp(m); r += r * (1 - m r); q = 127 r;
q += r * (127 - m q), each step one f32 operation (fused multiply-adds
round once). This restates those steps in exact rational arithmetic, with
the hardware reciprocal anywhere within one unit of 1/m, and checks that
the result is the correctly rounded quotient, and the exact one for the
only m whose quotient is representable (1/2 and 127/128). Host-only."""
import random
from fractions import Fraction as F


def _ulp(x):
    a = abs(F(x))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    return F(2) ** (e - 23)


def _rnd(x):
    """Round to the nearest f32, ties to even (normal range)."""
    x = F(x)
    if x == 0:
        return x
    u = _ulp(x)
    q, r = divmod(abs(x), u)
    if 2 * r > u or (2 * r == u and q % 2 == 1):
        q += 1
    return (1 if x > 0 else -1) * q * u


def _fma(a, b, c):
    return _rnd(F(a) * F(b) + F(c))


def _quotient(m, rcp):
    r = _fma(_fma(-m, rcp, 1), rcp, rcp)
    q = _rnd(127 * r)
    return _fma(_fma(-m, q, 127), r, q)


def _cases(m):
    r0 = _rnd(1 / m)
    return (r0 - _ulp(r0), r0, r0 + _ulp(r0))


def test_quotient_is_correctly_rounded():
    rng = random.Random(7)
    ms = [F(rng.randint(2 ** 23, 2 ** 24 - 1), 2 ** 24) for _ in range(1500)]
    ms += [F(1, 2), F(2 ** 24 - 1, 2 ** 24), F(127, 128), F(3, 4)]
    for m in ms:
        exact = F(127) / m
        want = _rnd(exact)
        for rcp in _cases(m):
            assert _quotient(m, rcp) == want, (m, rcp)


def test_representable_quotients_are_exact():
    # 127 / m is an f32 only for m = 1/2 (254) and m = 127/128 (128)
    for m, q in ((F(1, 2), 254), (F(127, 128), 128)):
        for rcp in _cases(m):
            assert _quotient(m, rcp) == q
