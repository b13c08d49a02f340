"""The group scale's division in the kernels, proved on the CPU.

The quantizer's scale is the correctly rounded fp32 quotient (max - min) / qmax (asymmetric,
qmax = 7, 15 or 255 for 3-, 4- and 8-bit codes) or max|w| / (h - 1) (symmetric: 3, 7, 127). The kernels form it without a division (`div_small` in
`csrc/common.hpp`): with y = RN(1/d), q0 = RN(x y), r = x - q0 d (one fma, exact) and
q1 = RN(q0 + r y) (one fma). This test replays those steps in exact arithmetic for every
fp32 significand x in [1, 2) and each divisor and checks q1 against the IEEE quotient
(numpy's float32 division), including ties. Powers of two scale every step exactly, so one
binade covers all normal x; the oracle keeps the plain division.
"""

from fractions import Fraction

import numpy as np
import pytest


def _fma_then_rn32_ok(q0, r, y, qref):
    """Whether RN32(q0 + r y), the exact value rounded once, equals qref: |v - qref| < ulp/2,
    with ties (|v - qref| = ulp/2) resolved to even and checked exactly."""
    ry = r.astype(np.float64) * np.float64(y)                   # exact (48 bits)
    diff = (q0.astype(np.float64) - qref.astype(np.float64)) + ry  # within 2^-53 relative
    ulp = np.spacing(qref).astype(np.float64)
    clear = np.abs(diff) < ulp / 2 * (1 - 2.0 ** -40)
    near = ~clear & (np.abs(np.abs(diff) - ulp / 2) <= ulp * 2.0 ** -40)
    bad = int((~clear & ~near).sum())
    for i in np.nonzero(near)[0]:
        v = Fraction(float(q0[i])) + Fraction(float(r[i])) * Fraction(float(y))
        q, u = Fraction(float(qref[i])), Fraction(float(ulp[i]))
        if abs(v - q) < u / 2:
            continue
        if abs(v - q) == u / 2 and (int(np.float32(qref[i]).view(np.int32)) & 1) == 0:
            continue  # a tie that rounds to the even qref
        bad += 1
    return bad


@pytest.mark.parametrize("d", [3, 7, 15, 127, 255])
def test_division_by_scale_divisor_is_correctly_rounded(d):
    m = np.arange(2 ** 23, 2 ** 24, dtype=np.int64)
    x = (m.astype(np.float64) * 2.0 ** -23).astype(np.float32)   # every significand, [1, 2)
    d32 = np.float32(d)
    y = np.float32(1.0) / d32                                     # RN(1/d)
    q0 = x * y                                                    # RN(x y)
    r64 = -q0.astype(np.float64) * d + x.astype(np.float64)       # x - q0 d, exact in fp64
    r = r64.astype(np.float32)
    assert np.array_equal(r.astype(np.float64), r64), "the residual must be exact in fp32"
    qref = x / d32                                                # IEEE quotient
    assert _fma_then_rn32_ok(q0, r, y, qref) == 0


def test_division_check_catches_a_missing_correction():
    """Planted mistake: RN(x y) alone (no fma correction) is not the IEEE quotient for every
    significand, and the check sees it."""
    m = np.arange(2 ** 23, 2 ** 24, dtype=np.int64)
    x = (m.astype(np.float64) * 2.0 ** -23).astype(np.float32)
    d32 = np.float32(15)
    q0 = x * (np.float32(1.0) / d32)
    zero = np.zeros_like(q0)
    assert _fma_then_rn32_ok(q0, zero, np.float32(0.0), x / d32) > 0
