"""The quantizers divide by the group scale S with a reciprocal and one
residual correction instead of a full IEEE division:

    y = RN(1/S), q0 = RN(x y), r = RN(x - S q0), q = RN(q0 + r y)

(see div_by_scale in the HIP sources).  This test proves, with exact
rational arithmetic, that q == RN(x / S) for every pair of significands the
quantizers can meet (x a bf16 value, S = RN(amax / 448) with amax a bf16
value).  The rounding depends only on the two significands as long as nothing
under- or overflows, so 128 x 128 pairs cover every normal-range case; the
kernels take the plain division whenever S < 2^-80."""
from fractions import Fraction as F


def rn32(fr: F) -> F:
    """Round a rational to the nearest binary32 value, ties to even (normal range)."""
    if fr == 0:
        return F(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    assert e >= -126
    ulp = F(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def test_reciprocal_correction_equals_ieee_division():
    mismatches = 0
    for ma in range(128):
        amax = F(128 + ma, 128)
        S = rn32(amax / 448)
        y = rn32(1 / S)
        for mx in range(128):
            x = F(128 + mx, 128)
            q0 = rn32(x * y)
            r = rn32(x - S * q0)
            q = rn32(r * y + q0)
            if q != rn32(x / S):
                mismatches += 1
    assert mismatches == 0
