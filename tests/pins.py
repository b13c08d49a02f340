"""Checks that pin a quantizer / searcher / linear to what the pages and the mathematics fix.

Each checker takes the outputs of some implementation (the oracle, or a deliberately
broken copy of it in the mutation tests) and returns a list of violations, computed
independently of that implementation: exact rational arithmetic (``fractions``),
brute force over all 16 codes, closed forms and invariants.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

GROUP = 128


def frac(x) -> Fraction:
    return Fraction(float(x))


def rne_fp16(v: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to IEEE binary16 (finite range)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1), clamped to the normal/subnormal boundary
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    m = a / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


def check_codes_nearest(w_scaled: np.ndarray, q: np.ndarray, z: np.ndarray, scale: np.ndarray,
                        qmax: int = 15) -> list:
    """P1: every unclamped code is the nearest one for the stored scale, in exact arithmetic.

    w_scaled: fp32 [N][K] values W*s (exact products); q uint8 [N][K]; z uint8 [N][G];
    scale fp16 [N][G]. A code may differ from the exact nearest only when the fp32
    quotient w'/sc lies within 2 fp32 ulps of a half-integer (then either neighbour
    is accepted) or when the nearest code falls outside 0..qmax (then the clamp).
    """
    bad = []
    N, K = q.shape
    group = K // np.asarray(scale).shape[1]
    for n in range(N):
        for k in range(K):
            j = k // group
            sc = frac(scale[n, j])
            zz = int(z[n, j])
            wv = frac(w_scaled[n, k])
            errs = [abs(wv - (c - zz) * sc) for c in range(qmax + 1)]
            best = min(errs)
            cands = {c for c in range(qmax + 1) if errs[c] == best}
            got = int(q[n, k])
            if got in cands:
                continue
            quot = wv / sc
            near_half = abs(quot - (Fraction(int(np.floor(float(quot)))) + Fraction(1, 2)))
            ulp = Fraction(2) ** (int(np.floor(np.log2(max(abs(float(quot)), 2.0 ** -20)))) - 23)
            if near_half <= 2 * ulp and abs(errs[got] - best) <= sc:
                continue
            bad.append((n, k, got, sorted(cands)))
    return bad


def check_scale_zero(w_scaled: np.ndarray, z: np.ndarray, scale: np.ndarray, ratio=None,
                     qmax: int = 15) -> list:
    """P2: closed form of the scale and the zero point from the group's extremes.

    sc_h must be the fp16 rounding of (mx - mn)/qmax up to the fp32 roundings on the
    way (a relative 2^-22 window), floored at 2^-14; z in [0, qmax]; when the zero is
    not clamped, -z*sc_h lies within sc_h/2 of mn. With ``ratio`` ([N][G], weight
    clipping) the extremes are r mx and r mn.
    """
    bad = []
    N, K = w_scaled.shape
    G = np.asarray(scale).shape[1]
    group = K // G
    for n in range(N):
        for j in range(G):
            g = w_scaled[n, j * group:(j + 1) * group]
            mx, mn = frac(g.max()), frac(g.min())
            if ratio is not None:
                r = frac(ratio[n, j])
                mx, mn = r * mx, r * mn
            exact = max((mx - mn) / qmax, Fraction(2) ** -14)
            lo_ = rne_fp16(exact * (1 - Fraction(1, 2 ** 22)))
            hi_ = rne_fp16(exact * (1 + Fraction(1, 2 ** 22)))
            sc = frac(scale[n, j])
            if not (lo_ <= sc <= hi_):
                bad.append(("scale", n, j, float(sc), float(exact)))
                continue
            zz = int(z[n, j])
            if not (0 <= zz <= qmax):
                bad.append(("zero-range", n, j, zz))
                continue
            ideal = -mn / sc
            if 0 <= ideal <= qmax and abs(-zz * sc - mn) > sc / 2 + sc * Fraction(1, 2 ** 20):
                bad.append(("zero", n, j, zz, float(ideal)))
    return bad


def exact_search_error(X16: np.ndarray, W16: np.ndarray, s16: np.ndarray, q, z, scale) -> Fraction:
    """P7: err = sum_t sum_n (sum_k X_tk D_nk)^2 with D = W - (q - z) sc / s, exactly."""
    T, K = X16.shape
    N = W16.shape[0]
    group = K // np.asarray(scale).shape[1]
    total = Fraction(0)
    for n in range(N):
        D = []
        for k in range(K):
            j = k // group
            what = (int(q[n, k]) - int(z[n, j])) * frac(scale[n, j]) / frac(s16[k])
            D.append(frac(W16[n, k]) - what)
        for t in range(T):
            e = sum((frac(X16[t, k]) * D[k] for k in range(K)), Fraction(0))
            total += e * e
    return total


def exact_group_errors(X16: np.ndarray, W16: np.ndarray, s16, q, z, scale) -> list:
    """Weight clipping: err[n][g] = sum_t (sum_{k in g} X_tk D_nk)^2, D = W - (q - z) sc / s,
    exactly (s16 None means s = 1)."""
    T, K = X16.shape
    N = W16.shape[0]
    G = np.asarray(scale).shape[1]
    group = K // G
    out = []
    for n in range(N):
        row = []
        for j in range(G):
            ks = range(j * group, (j + 1) * group)
            D = {}
            for k in ks:
                sk = frac(s16[k]) if s16 is not None else Fraction(1)
                D[k] = frac(W16[n, k]) - (int(q[n, k]) - int(z[n, j])) * frac(scale[n, j]) / sk
            tot = Fraction(0)
            for t in range(T):
                e = sum((frac(X16[t, k]) * D[k] for k in ks), Fraction(0))
                tot += e * e
            row.append(tot)
        out.append(row)
    return out
