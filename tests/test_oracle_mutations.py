"""Planted mistakes: broken copies of oracle steps must be caught by the pins.

Each mutant changes one step of the quantizer / search in a plausible way (a sign,
a rounding function, a constant, an index, a dropped factor); the checker that pins
that step must report it. The real oracle passes the same checkers in
test_oracle_pins.py.
"""

from fractions import Fraction

import numpy as np

import oracle
import synthetic_inputs as si
from tests import pins


def _quant(W16, s16=None, *, zero_sign=-1.0, rounder=np.rint, levels=15.0, use_stored_scale=True):
    w = W16.astype(np.float32)
    if s16 is not None:
        w = w * s16.astype(np.float32)[None, :]
    N, K = w.shape
    wg = w.reshape(N, K // 128, 128)
    mx, mn = wg.max(2), wg.min(2)
    sc = np.maximum((mx - mn) / np.float32(levels), np.float32(2.0 ** -14))
    sch = sc.astype(np.float16)
    scf = sch.astype(np.float32) if use_stored_scale else sc
    z = np.clip(rounder(np.float32(zero_sign) * mn / scf), 0, 15)
    q = np.clip(rounder(wg / scf[..., None]) + z[..., None], 0, 15)
    return w, q.astype(np.uint8).reshape(N, K), z.astype(np.uint8), sch


W = si.weights(2, 256, offset=50)


def test_reference_quantizer_passes():
    w, q, z, sc = _quant(W)
    assert not pins.check_codes_nearest(w, q, z, sc)
    assert not pins.check_scale_zero(w, z, sc)


def test_zero_point_sign_mutant_caught():
    w, q, z, sc = _quant(W, zero_sign=+1.0)
    assert pins.check_scale_zero(w, z, sc) or pins.check_codes_nearest(w, q, z, sc)


def test_floor_rounding_mutant_caught():
    w, q, z, sc = _quant(W, rounder=np.floor)
    assert pins.check_codes_nearest(w, q, z, sc)


def test_wrong_level_count_mutant_caught():
    w, q, z, sc = _quant(W, levels=16.0)
    assert pins.check_scale_zero(w, z, sc)


def test_unrounded_scale_mutant_caught_on_codes():
    # codes rounded against the fp32 scale instead of the stored fp16 one
    w, q, z, sc = _quant(si.weights(8, 512, offset=51), use_stored_scale=False)
    ref = oracle.quantize_groups(si.weights(8, 512, offset=51))
    assert not np.array_equal(q, ref["q"]) or not np.array_equal(z, ref["z"])


def test_sequential_nibble_order_mutant_caught():
    q = np.arange(8 * 16, dtype=np.uint8).reshape(1, 128) % 16
    qw, _, _ = oracle.pack(q, np.zeros((1, 1), np.uint8), np.ones((1, 1), np.float16))
    word = 0
    for j in range(8):                     # mutant: nibble j holds channel j
        word |= int(q[0, j]) << (4 * j)
    assert word != int(qw[0, 0])
    assert int(qw[0, 0]) == 0x75316420     # hand-derived: nibbles hold channels 0,2,4,6,1,3,5,7


def test_dropped_inverse_scale_mutant_caught():
    X = si.activations(2, 128, offset=52)
    Wt = si.weights(1, 128, offset=52)
    r = oracle.search_errors(X, Wt, n_grid=3)
    i = 2
    qz = oracle.quantize_groups(Wt, r["s16"][i])
    exact = pins.exact_search_error(X, Wt, r["s16"][i], qz["q"], qz["z"], qz["scale"])
    # mutant: forget to divide the dequantized weight by s
    deq = oracle.dequantize(qz["q"], qz["z"], qz["scale"])
    E = X.astype(np.float64) @ (Wt.astype(np.float64) - deq).T
    mutant = float(np.sum(E * E))
    assert abs(mutant - float(exact)) > 1e-6 * float(exact)
    assert abs(r["err"][i] - float(exact)) <= 1e-12 * float(exact)


def test_signed_mean_mutant_caught():
    X = np.array([[1.0, -2.0], [3.0, 0.5]], dtype=np.float16)
    mutant = X.astype(np.float64).mean(axis=0)
    exact = [Fraction(4, 2), Fraction(5, 4)]
    assert [float(v) for v in exact] != mutant.tolist()
    assert oracle.activation_mean_abs(X)[0].tolist() == [float(v) for v in exact]


def test_3bit_plane_mutants_caught():
    """Plausible 3-bit layout slips differ from the hand-derived words: the two channels of a
    pair in adjacent fields instead of the two halves, the planes swapped (bit 2 with the low
    field), or the high bits one per channel in channel order."""
    q = (np.arange(128, dtype=np.uint8) * 5 % 8).reshape(1, 128)
    qw, _, _ = oracle.pack(q, np.zeros((1, 1), np.uint8), np.ones((1, 1), np.float16), w_bit=3)
    # hand-derived: low word 0 = bits 0-1 of channels 0,2,..,14 (low half), 1,3,..,15 (high)
    lo0 = sum((int(q[0, 2 * f]) & 3) << (2 * f) for f in range(8)) | \
        sum((int(q[0, 2 * f + 1]) & 3) << (16 + 2 * f) for f in range(8))
    hi0 = sum((int(q[0, 2 * p]) >> 2) << p for p in range(16)) | \
        sum((int(q[0, 2 * p + 1]) >> 2) << (16 + p) for p in range(16))
    assert int(qw[0, 0]) == lo0 and int(qw[0, 8]) == hi0
    adjacent = sum((int(q[0, c]) & 3) << (2 * c) for c in range(16))
    assert adjacent != int(qw[0, 0])
    swapped = sum((int(q[0, 2 * f]) >> 2) << (2 * f) for f in range(8))
    assert swapped != int(qw[0, 0])
    in_order = sum((int(q[0, c]) >> 2) << c for c in range(32))
    assert in_order != int(qw[0, 8])
