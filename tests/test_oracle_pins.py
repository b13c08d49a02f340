"""CPU pins of the oracle against what the AWQ pages and the mathematics fix.

Each test names the passage or the mathematical fact it holds the oracle to. None
of these tests re-types the oracle's formulas: they use hand-worked values
(tests/golden/hand_worked.json), exact rational arithmetic, brute force over the
16 codes, closed forms and invariants.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from tests import pins

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


def golden_group_row(g):
    w = np.full(128, g["fill"], dtype=np.float16)
    for k, v in g["values"].items():
        w[int(k)] = v
    return w


# ----------------------------------------------------------------- hand-worked values
@pytest.mark.parametrize("g", GOLDEN["groups"], ids=[g["name"] for g in GOLDEN["groups"]])
def test_golden_group(g):
    """Hand-worked groups ('AWQ量化实战' §2.3; 'GPTQ与AWQ' 4-bit + scale + zero point)."""
    W = golden_group_row(g)[None, :]
    r = oracle.quantize_groups(W)
    assert r["scale"].view(np.uint16)[0, 0] == int(g["scale_bits"], 16)
    assert r["z"][0, 0] == g["zero"]
    for k in range(128):
        want = g["codes"].get(str(k), g["fill_code"])
        assert r["q"][0, k] == want, (k, r["q"][0, k], want)


def test_golden_packing():
    p = GOLDEN["packing"]
    q = np.zeros((1, 3 * 128), dtype=np.uint8)
    q[0, :8] = p["codes_k0_to_k7"]
    z = np.array([p["zeros_groups"]], dtype=np.uint8)
    sc = np.ones((1, 3), dtype=np.float16)
    qw, _, zb = oracle.pack(q, z, sc)
    assert int(qw[0, 0]) == int(p["word"], 16)
    assert [int(b) for b in zb[0]] == [int(b, 16) for b in p["zeros_bytes"]]


def test_golden_activation_mean():
    g = GOLDEN["activation_mean"]
    a, flags = oracle.activation_mean_abs(np.array(g["X"], dtype=np.float16))
    assert flags == 0
    assert a.tolist() == g["a"]


def test_golden_candidate_scales():
    g = GOLDEN["candidate_scales"]
    _, s16, _ = oracle.candidate_scales(np.array(g["a"]), g["n_grid"])
    assert s16.astype(np.float64).tolist() == g["s"]


def test_golden_search_error():
    """One token e_0 through the 'straddling zero' group: err = D_0^2 = 2^-24, worked by hand."""
    W = golden_group_row(GOLDEN["groups"][0])[None, :]
    X = np.zeros((1, 128), dtype=np.float16)
    X[0, 0] = 1.0
    r = oracle.search_errors(X, W, n_grid=1)
    assert r["err"][0] == GOLDEN["search_error"]["err"]


# ----------------------------------------------------------------- a1 statistic
def test_activation_mean_exact_vs_rationals():
    """a_k = (1/T) sum |x|: compare with exact rational sums, correctly rounded to fp64."""
    g = np.random.default_rng(1)
    bits = g.integers(0, 0x7C00, size=(37, 9), dtype=np.uint16)   # every finite fp16 magnitude
    sign = g.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15
    X = (bits | sign).view(np.float16)
    a, flags = oracle.activation_mean_abs(X)
    assert flags == 0
    for k in range(X.shape[1]):
        exact = sum((abs(Fraction(float(v))) for v in X[:, k]), Fraction(0)) / X.shape[0]
        assert a[k] == float(exact)


def test_activation_mean_extreme_and_order():
    """Largest calibration set, largest fp16 magnitudes plus subnormals: still exact and order-free."""
    T = oracle.awq_oracle.MAX_CALIB_TOKENS
    X = np.full((T, 2), 65504.0, dtype=np.float16)
    X[::3, 1] = np.float16(2.0 ** -24)
    X[1::7, 0] = -X[1::7, 0]
    a, _ = oracle.activation_mean_abs(X)
    exact0 = Fraction(65504) * T / T
    n_sub = len(range(0, T, 3))
    exact1 = (Fraction(65504) * (T - n_sub) + Fraction(1, 2 ** 24) * n_sub) / T
    assert a[0] == float(exact0) and a[1] == float(exact1)
    perm = np.random.default_rng(2).permutation(T)
    a2, _ = oracle.activation_mean_abs(X[perm])
    assert np.array_equal(a, a2)


def test_activation_nonfinite_flag():
    X = np.ones((4, 8), dtype=np.float16)
    X[2, 3] = np.inf
    assert oracle.activation_mean_abs(X)[1] & oracle.FLAG_NONFINITE_INPUT


# ----------------------------------------------------------------- a2 candidate scales
def test_fp16_conversion_is_single_rounding():
    """fp64 -> fp16 must round once (RNE); going through fp32 would double-round."""
    vals = [1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
            2.0 ** -14 * (1 + 2.0 ** -11 + 2.0 ** -45), 65519.99, 0.1, 1 / 3]
    for v in vals:
        got = Fraction(float(np.float64(v).astype(np.float16)))
        assert got == pins.rne_fp16(Fraction(v)), v


def test_candidate_scales_closed_forms():
    """alpha_0 = 0 gives s = 1 (plain RTN, 'AWQ量化实战' §1.1); powers of two are exact."""
    a = np.array([4096.0, 0.25, 1.0, 2.0 ** -30, 37.5])
    alpha, s16, s64 = oracle.candidate_scales(a, 20)
    assert alpha.tolist() == [i / 20 for i in range(20)]
    assert np.all(s16[0] == 1.0)
    # 4096^(i/20) = 2^(12 i / 20): exact powers of two at i = 5, 10, 15
    assert s16[5, 0] == 8.0 and s16[10, 0] == 64.0 and s16[15, 0] == 512.0
    assert s16[10, 1] == 0.25 ** 0.5
    assert np.all(s16[:, 2] == 1.0)
    # the floor: a below 2^-14 behaves like 2^-14
    _, s_floor, _ = oracle.candidate_scales(np.array([2.0 ** -14]), 20)
    assert np.array_equal(s16[:, 3], s_floor[:, 0])
    # monotone in alpha: increasing for a > 1, decreasing for a < 1
    assert np.all(np.diff(s16[:, 4].astype(np.float64)) >= 0)
    assert np.all(np.diff(s16[:, 1].astype(np.float64)) <= 0)
    # each stored value is the RNE fp16 of a value within 1e-15 relative of the real power
    for i in range(20):
        for k in range(a.size):
            real = max(a[k], 2.0 ** -14) ** (i / 20)
            assert abs(s64[i, k] - real) <= 1e-15 * real


# ----------------------------------------------------------------- a3 quantizer
def _scaled(W16, s16):
    w = W16.astype(np.float32)
    return w if s16 is None else w * s16.astype(np.float32)[None, :]


@pytest.mark.parametrize("use_s", [False, True])
def test_codes_are_nearest_bruteforce(use_s):
    """P1: each code is the nearest of the 16 levels (exact arithmetic) for the stored scale."""
    W = si.weights(3, 256, offset=11)
    W[0, 5] = 0.3                                  # plant a few special values
    W[1, :128] = np.float16(0.01)                  # one constant group
    s = None
    if use_s:
        a, _ = oracle.activation_mean_abs(si.activations(16, 256, offset=3))
        s = oracle.candidate_scales(a, 20)[1][13]
    r = oracle.quantize_groups(W, s)
    bad = pins.check_codes_nearest(_scaled(W, s), r["q"], r["z"], r["scale"])
    assert not bad, bad[:5]


def test_scale_and_zero_closed_form():
    """P2: sc_h = fp16((mx - mn)/15) (up to fp32 roundings), 0 <= z <= 15, -z sc_h ~ mn."""
    W = si.weights(4, 512, offset=12)
    W[2, 128:256] = np.abs(W[2, 128:256]) + np.float16(0.05)  # a group that does not straddle 0
    r = oracle.quantize_groups(W)
    assert not pins.check_scale_zero(_scaled(W, None), r["z"], r["scale"])


def test_rtn_is_unit_scale():
    """P4: s = 1 reproduces plain round-to-nearest ('AWQ量化实战' §1.1)."""
    W = si.weights(5, 384, offset=13)
    a = oracle.quantize_groups(W)
    b = oracle.quantize_groups(W, np.ones(384, dtype=np.float16))
    for key in ("q", "z"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["scale"].view(np.uint16), b["scale"].view(np.uint16))


def test_power_of_two_equivariance():
    """P5: min/max affine quantization commutes with exact power-of-two scaling."""
    W = si.weights(4, 256, offset=14)
    base = oracle.quantize_groups(W)
    for e in (-3, 2, 5):
        r = oracle.quantize_groups((W.astype(np.float32) * 2.0 ** e).astype(np.float16))
        assert np.array_equal(base["q"], r["q"]) and np.array_equal(base["z"], r["z"])
        assert np.array_equal(base["scale"].astype(np.float64) * 2.0 ** e, r["scale"].astype(np.float64))


def test_group_locality():
    """P6: a group's codes, scale and zero depend on its own 128 values only ('AWQ量化实战' §2.3)."""
    W = si.weights(3, 512, offset=15)
    base = oracle.quantize_groups(W)
    W2 = W.copy()
    W2[1, 256:384] = (W2[1, 256:384].astype(np.float32) * 3 + 0.01).astype(np.float16)
    r = oracle.quantize_groups(W2)
    changed_q = np.argwhere(np.any(base["q"] != r["q"], axis=0)).ravel()
    assert changed_q.size and changed_q.min() >= 256 and changed_q.max() < 384
    diff_groups = np.argwhere(base["scale"] != r["scale"])
    assert diff_groups.tolist() == [[1, 2]]


def test_scale_clamp_flag():
    W = np.zeros((1, 128), dtype=np.float16)
    W[0, 0], W[0, 1] = -60000.0, 60000.0
    s = np.full(128, 20.0, dtype=np.float16)
    r = oracle.quantize_groups(W, s)
    assert r["flags"] & oracle.FLAG_SCALE_CLAMPED
    assert float(r["scale"][0, 0]) == 65504.0


# ----------------------------------------------------------------- a4 packing
def test_pack_roundtrip_odd_groups():
    g = np.random.default_rng(5)
    for K in (128, 384, 1024):
        q = g.integers(0, 16, size=(3, K), dtype=np.uint8)
        z = g.integers(0, 16, size=(3, K // 128), dtype=np.uint8)
        sc = g.standard_normal((3, K // 128)).astype(np.float16)
        qw, s2, zb = oracle.pack(q, z, sc)
        assert qw.dtype == np.uint32 and qw.shape == (3, K // 8)
        assert zb.shape == (3, (K // 128 + 1) // 2)
        q2, z2, s3 = oracle.unpack(qw, s2, zb, K)
        assert np.array_equal(q, q2) and np.array_equal(z, z2) and np.array_equal(sc, s3)
    if (K // 128) % 2:
        assert np.all(zb[:, -1] >> 4 == 0)


def test_one_hot_extracts_dequantized_column():
    """P3: x = e_k returns (q_nk - z) sc exactly, from the packed words read by hand."""
    W = si.weights(6, 256, offset=16)
    qw, sc, zb, _ = oracle.quantize_pack(W)
    for k in (0, 7, 8, 129, 255):
        X = np.zeros((1, 256), dtype=np.float16)
        X[0, k] = 1.0
        y, bound = oracle.linear_reference(X, qw, sc, zb, 256)
        nibble = (0, 4, 1, 5, 2, 6, 3, 7)[k % 8]   # channel 8w + (0,2,4,6,1,3,5,7)[j] sits in nibble j
        for n in range(6):
            code = (int(qw[n, k // 8]) >> (4 * nibble)) & 0xF
            j = k // 128
            zero = (int(zb[n, j // 2]) >> (4 * (j % 2))) & 0xF
            assert y[0, n] == (code - zero) * float(sc[n, j])
            assert bound[0, n] == abs(y[0, n])


# ----------------------------------------------------------------- a5/a6 search
def test_search_error_exact_rationals():
    """P7: fp64 errors agree with exact rational errors on tiny problems, same argmin."""
    for (T, N, K, off) in ((3, 2, 128, 0), (2, 1, 256, 1)):
        X = si.activations(T, K, offset=20 + off)
        W = si.weights(N, K, offset=20 + off)
        r = oracle.search_errors(X, W, n_grid=4)
        exact = []
        for i in range(4):
            qz = oracle.quantize_groups(W, r["s16"][i])
            exact.append(pins.exact_search_error(X, W, r["s16"][i], qz["q"], qz["z"], qz["scale"]))
        for i in range(4):
            assert abs(r["err"][i] - float(exact[i])) <= 1e-12 * float(exact[i])
        assert int(np.argmin(r["err"])) == min(range(4), key=lambda i: (exact[i], i))


def test_search_never_worse_than_rtn():
    """P8: alpha = 0 (plain RTN) is on the grid, so the chosen error cannot exceed it."""
    X = si.activations(64, 512, offset=30)
    W = si.weights(64, 512, offset=30)
    r = oracle.search_scales(X, W)
    assert r["err"][r["best_idx"]] <= r["err"][0]
    assert r["best_idx"] > 0 and r["err"][r["best_idx"]] < r["err"][0]  # heavy tail helps (sanity)


def test_unit_activations_tie_to_first():
    """P9: |x| = 1 everywhere -> a = 1 -> s = 1 for every alpha -> equal errors -> index 0."""
    g = np.random.default_rng(7)
    X = np.where(g.integers(0, 2, size=(8, 256)) == 1, 1.0, -1.0).astype(np.float16)
    W = si.weights(16, 256, offset=31)
    r = oracle.search_scales(X, W)
    assert np.all(r["err"] == r["err"][0])
    assert r["best_idx"] == 0 and np.all(r["s_best"] == 1.0)


def test_search_result_is_pack_with_best_scale():
    X = si.activations(32, 256, offset=32)
    W = si.weights(8, 256, offset=32)
    r = oracle.search_scales(X, W)
    qw, sc, zb, _ = oracle.quantize_pack(W, r["s16"][r["best_idx"]])
    assert np.array_equal(qw, r["qweight"]) and np.array_equal(zb, r["zeros"])


# ----------------------------------------------------------------- a7/a8 linear
def test_linear_zero_and_row_independence():
    """P10: X = 0 gives 0; an M-row batch equals M single-row products."""
    W = si.weights(9, 384, offset=40)
    qw, sc, zb, _ = oracle.quantize_pack(W)
    y0, b0 = oracle.linear_reference(np.zeros((2, 384), dtype=np.float16), qw, sc, zb, 384)
    assert np.all(y0 == 0) and np.all(b0 == 0)
    X = si.activations(5, 384, offset=40)
    y, _ = oracle.linear_reference(X, qw, sc, zb, 384)
    for m in range(5):
        ym, _ = oracle.linear_reference(X[m:m + 1], qw, sc, zb, 384)
        assert np.allclose(ym[0], y[m], rtol=1e-14, atol=1e-14)


def test_linear_reference_vs_rationals():
    W = si.weights(3, 128, offset=41)
    qw, sc, zb, _ = oracle.quantize_pack(W)
    X = si.activations(2, 128, offset=41)
    y, bound = oracle.linear_reference(X, qw, sc, zb, 128)
    q, z, s = oracle.unpack(qw, sc, zb, 128)
    for m in range(2):
        for n in range(3):
            terms = [Fraction(float(X[m, k])) * (int(q[n, k]) - int(z[n, 0])) * Fraction(float(s[n, 0]))
                     for k in range(128)]
            assert abs(y[m, n] - float(sum(terms))) <= 1e-14 * float(sum(abs(t) for t in terms))
            assert abs(bound[m, n] - float(sum(abs(t) for t in terms))) <= 1e-14 * bound[m, n]


# ----------------------------------------------------------------- hazards and format
def test_midpoint_hazard_detector():
    """P11: values next to an fp16 rounding midpoint are detected; ordinary values are not."""
    mid = 1.0 + 2.0 ** -11
    d = oracle.fp16_midpoint_distance(np.array([mid * (1 + 2.0 ** -50), 1.3, mid]))
    assert d[0] < 2.0 ** -40 and d[1] > 1e-4 and d[2] == 0.0


def test_relative_gap():
    assert oracle.relative_gap(np.array([3.0, 1.0, 1.5])) == 0.5
    assert oracle.relative_gap(np.array([2.0, 2.0])) == 0.0


def test_format_size_matches_70b_figure():
    """P13: 80 Llama-2-70B layers pack to ~35 GB ('AWQ量化技术Skill': 70B 140 GB -> 35 GB)."""
    per_layer = sum(oracle.packed_bytes(n, k) for n, k in si.LLAMA2_70B_LINEARS.values())
    total = per_layer * si.LLAMA2_70B_LAYERS
    assert total == 68_451_041_280 * 133 // 256   # 0.51953125 B per weight = 35.56 GB
    assert 33e9 < total < 37e9
    assert oracle.packed_bytes(4096, 4096) * 8 == 4096 * 4096 * 4 + 4096 * 32 * 16 + 4096 * 16 * 8


# ----------------------------------------------------------------- fused MLP (gate|up)
def test_silu_matches_library_logistic():
    """SiLU(v) = v * logistic(v), against scipy's expit over the fp16 range and beyond."""
    from scipy.special import expit
    v = np.concatenate([np.linspace(-60, 60, 20001), [-1000.0, -745.5, 0.0, 1e-30, 65504.0]])
    ref = v * expit(v)
    got = oracle.silu(v)
    assert np.all(np.abs(got - ref) <= 4 * np.finfo(np.float64).eps * np.abs(ref) + 1e-300)


def test_silu_odd_part_identity_and_derivative_bound():
    """SiLU(-v) = SiLU(v) - v (logistic symmetry); max |SiLU'| is just below SILU_DMAX."""
    v = np.linspace(0, 40, 4001)
    assert np.allclose(oracle.silu(-v), oracle.silu(v) - v, rtol=0, atol=1e-13)
    x = np.linspace(-30, 30, 600001)
    d = np.diff(oracle.silu(x)) / np.diff(x)
    assert 1.09 < np.max(np.abs(d)) <= oracle.SILU_DMAX


def _gate_up_case(nh=6, K=256, off=90):
    W = si.weights(2 * nh, K, offset=off)
    qw, sc, zb, _ = oracle.quantize_pack(W)
    q, z, scale = oracle.unpack(qw, sc, zb, K)
    return qw, sc, zb, oracle.dequantize(q, z, scale)


def test_gated_silu_gate_rows_first():
    """One-hot x = e_k: h_n = SiLU(deq_gate[n, k]) * deq_up[n, k], gate rows first."""
    import math
    nh, K = 6, 256
    qw, sc, zb, deq = _gate_up_case(nh, K)
    ks = [0, 1, 127, 128, 255]
    X = np.zeros((len(ks), K), dtype=np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1.0
    h, g, u, bg, bu = oracle.gated_silu_reference(X, qw, sc, zb, K)
    assert h.shape == (len(ks), nh)
    for m, k in enumerate(ks):
        for n in range(nh):
            a, b = float(deq[n, k]), float(deq[nh + n, k])
            assert h[m, n] == pytest.approx(a / (1.0 + math.exp(-a)) * b, rel=1e-15, abs=1e-300)
            assert bg[m, n] == abs(a) and bu[m, n] == abs(b)
    # mutant: up rows first
    swapped = oracle.silu(u) * g
    assert not np.allclose(swapped, h, rtol=1e-6, atol=0)


def test_gated_silu_tolerance_covers_linear_errors():
    """Any g', u' within the linear tolerance, with one fp16 rounding of SiLU(g') u', passes;
    a result off by a few percent does not."""
    rng = np.random.default_rng(5)
    qw, sc, zb, _ = _gate_up_case(64, 512, off=91)
    X = si.activations(8, 512, offset=91)
    h, g, u, bg, bu = oracle.gated_silu_reference(X, qw, sc, zb, 512)
    for _ in range(20):
        g2 = g + rng.uniform(-1, 1, g.shape) * 2e-3 * bg
        u2 = u + rng.uniform(-1, 1, u.shape) * 2e-3 * bu
        h2 = (oracle.silu(g2) * u2).astype(np.float16).astype(np.float64)
        assert oracle.gated_silu_within_tolerance(h2, g, u, bg, bu).all()
    assert not oracle.gated_silu_within_tolerance(h * 1.05, g, u, bg, bu).all()


# ----------------------------------------------------------------- equivalent transform
def test_inverse_scale_hand_worked_and_axes():
    """fp16(A / s): hand-worked quotients (exact, and correctly rounded), both axes."""
    A = np.array([[1.0, 3.0, -0.5], [6.0, 1.0, 65504.0]], dtype=np.float16)
    s_cols = np.array([2.0, 3.0, 0.25], dtype=np.float16)
    out, flags = oracle.apply_inverse_scale(A, s_cols, axis=1)
    # 1/2 = 0.5, 3/3 = 1, -0.5/0.25 = -2; 6/2 = 3, 1/3 -> fp16 0x3555 (0.333251953125),
    # 65504/0.25 = 262016 > 65504 -> inf (overflow flagged)
    assert out[0].tolist() == [0.5, 1.0, -2.0]
    assert out[1, 0] == 3.0 and out[1, 1].view(np.uint16) == 0x3555 and np.isinf(out[1, 2])
    assert flags == oracle.FLAG_OVERFLOW
    s_rows = np.array([4.0, 0.5], dtype=np.float16)
    out0, f0 = oracle.apply_inverse_scale(A[:, :2], s_rows, axis=0)
    assert out0.tolist() == [[0.25, 0.75], [12.0, 2.0]] and f0 == 0


def test_inverse_scale_is_correctly_rounded():
    """Against exact rational arithmetic: |fp16 result - a/s| <= half an fp16 ulp, ties even."""
    rng = np.random.default_rng(3)
    A = (rng.standard_normal((64, 256)) * 3).astype(np.float16)
    s = np.exp(rng.uniform(-3, 3, 256)).astype(np.float16)
    out, _ = oracle.apply_inverse_scale(A, s, axis=1)
    for r in range(0, 64, 7):
        for k in range(0, 256, 5):
            exact = Fraction(float(A[r, k])) / Fraction(float(s[k]))
            got = Fraction(float(out[r, k]))
            h = np.float16(out[r, k])
            ulp = Fraction(float(np.spacing(np.abs(h)))) if h != 0 else Fraction(2) ** -24
            assert abs(got - exact) <= ulp / 2


def test_equivalent_transform_identity_without_quantization():
    """X W^T = (X diag(1/s)) (W diag(s))^T exactly when s are powers of two."""
    X = si.activations(4, 256, offset=95)
    W = si.weights(8, 256, offset=95)
    s = (2.0 ** np.random.default_rng(4).integers(0, 4, 256)).astype(np.float16)
    Xs, _ = oracle.apply_inverse_scale(X, s, axis=1)
    Ws = (W.astype(np.float64) * s.astype(np.float64)).astype(np.float16)
    lhs = X.astype(np.float64) @ W.astype(np.float64).T
    rhs = Xs.astype(np.float64) @ Ws.astype(np.float64).T
    # both sides exact (no fp16 underflow of X / s, W * s stays in range)
    assert np.all(Xs.astype(np.float64) * s == X.astype(np.float64))
    assert np.all(Ws.astype(np.float64) / s == W.astype(np.float64))
    assert np.array_equal(lhs, rhs)


# ----------------------------------------------------------------- weight clipping
def test_clip_grid_and_ratio_one_is_plain_quantization():
    """r_i = (200 - i) / 200 in fp32; a one-point grid (r = 1) packs exactly as without clipping."""
    r = oracle.clip_ratios(200, 100)
    assert r[0] == 1.0 and r[1] == np.float32(0.995) and r[-1] == np.float32(0.505)
    assert np.all(np.diff(r.astype(np.float64)) < 0)
    X = si.activations(16, 256, offset=110)
    W = si.weights(6, 256, offset=110)
    a, _ = oracle.activation_mean_abs(X)
    s = oracle.candidate_scales(a, 20)[1][7]
    c = oracle.clip_search(X, W, s, 200, 1)
    qw, sc, zb, _ = oracle.quantize_pack(W, s)
    assert np.all(c["idx"] == 0)
    assert np.array_equal(c["qweight"], qw) and np.array_equal(c["zeros"], zb)
    assert np.array_equal(c["scales"].view(np.uint16), sc.view(np.uint16))


def test_clipped_codes_nearest_and_ranges():
    """Shrunk ranges: codes are the nearest in the clipped grid (weights beyond it take the
    end codes), and scale / zero follow the closed form on r mx, r mn."""
    W = si.weights(4, 256, offset=111)
    s = np.exp(np.random.default_rng(6).uniform(-1, 1, 256)).astype(np.float16)
    ratio = oracle.clip_ratios(200, 100)[np.random.default_rng(7).integers(0, 100, (4, 2))]
    qz = oracle.quantize_groups(W, s, ratio)
    w = W.astype(np.float32) * s.astype(np.float32)
    assert not pins.check_codes_nearest(w, qz["q"], qz["z"], qz["scale"])
    assert not pins.check_scale_zero(w, qz["z"], qz["scale"], ratio)
    # mutant: the range shrunk from the top only
    mx_only = oracle.quantize_groups(W, s, None)
    assert pins.check_scale_zero(w, mx_only["z"], mx_only["scale"], ratio)


def test_clip_errors_exact_and_separable():
    """Per-group errors against exact rational arithmetic; a change in one group leaves the
    other group's errors untouched; the choice is the first minimum."""
    X = si.activations(3, 256, offset=112)
    W = si.weights(2, 256, offset=112)
    s = np.exp(np.random.default_rng(8).uniform(-0.5, 0.5, 256)).astype(np.float16)
    err = oracle.clip_errors(X, W, s, 200, 5)
    for i, r in enumerate(oracle.clip_ratios(200, 5)):
        qz = oracle.quantize_groups(W, s, np.full((2, 2), r, dtype=np.float32))
        ex = pins.exact_group_errors(X, W, s, qz["q"], qz["z"], qz["scale"])
        for n in range(2):
            for g in range(2):
                assert abs(err[i, n, g] - float(ex[n][g])) <= 1e-12 * float(ex[n][g])
    W2 = W.copy()
    W2[:, 128:] = si.weights(2, 128, offset=113)
    err2 = oracle.clip_errors(X, W2, s, 200, 5)
    assert np.array_equal(err2[:, :, 0], err[:, :, 0]) and not np.array_equal(err2[:, :, 1], err[:, :, 1])
    c = oracle.clip_search(X, W, s, 200, 5)
    for n in range(2):
        for g in range(2):
            e = err[:, n, g]
            assert c["idx"][n, g] == int(np.flatnonzero(e == e.min())[0])


def test_clipping_an_outlier_the_tokens_never_see():
    """Worked case: weights spread over [0.0024, 0.3] plus one outlier at 1.5 on a channel the
    calibration tokens leave at zero. Min/max puts the step at (1.5 - 0.0024)/15 ~ 0.1; at the
    grid's smallest ratio 0.505 the range is both ends times 0.505 and the step half as large,
    so the weights the tokens use are rounded about twice as finely (squared error about a
    quarter) while the clipped outlier costs nothing; the search keeps the smallest error."""
    W = (np.arange(128) * (0.3 / 127)).astype(np.float16)[None, :]
    W[0, 0] = 1.5
    X = si.activations(4, 128, offset=114)
    X[:, 0] = 0
    err = oracle.clip_errors(X, W, None, 200, 100)[:, 0, 0]
    w1 = float(W[0, 1])
    qz0 = oracle.quantize_groups(W, None, np.ones((1, 1), np.float32))
    qz1 = oracle.quantize_groups(W, None, np.full((1, 1), 0.505, np.float32))
    assert float(qz0["scale"][0, 0]) == pytest.approx((1.5 - w1) / 15, rel=2 ** -10)  # fp16 step
    assert float(qz1["scale"][0, 0]) == pytest.approx(0.505 * (1.5 - w1) / 15, rel=2 ** -10)
    assert qz0["z"][0, 0] == 0 and qz1["z"][0, 0] == 0 and qz1["q"][0, 0] == 15
    assert err[-1] < err[0] / 3
    assert oracle.clip_search(X, W, None, 200, 100)["idx"][0, 0] == int(np.argmin(err))


# ----------------------------------------------------------------- symmetric codes
def test_symmetric_hand_worked_group():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))["symmetric_group"]
    W = np.full((1, 128), g["fill"], dtype=np.float16)
    for k, v in g["values"].items():
        W[0, int(k)] = v
    r = oracle.quantize_groups(W, zero_point=False)
    assert hex(int(r["scale"].view(np.uint16)[0, 0])) == g["scale_bits"]
    assert int(r["z"][0, 0]) == g["zero"]
    for k, c in g["codes"].items():
        assert int(r["q"][0, int(k)]) == c
    assert int(r["q"][0, 100]) == g["fill_code"]


def _check_symmetric_scale(w, z, scale):
    """sc_h = fp16(max |w'| / 7) up to the fp32 division's rounding, floored at 2^-14; z = 8."""
    bad = []
    for n in range(w.shape[0]):
        for j in range(w.shape[1] // 128):
            grp = w[n, j * 128:(j + 1) * 128]
            amax = max(Fraction(float(abs(grp.max()))), Fraction(float(abs(grp.min()))))
            exact = max(amax / 7, Fraction(2) ** -14)
            lo_ = pins.rne_fp16(exact * (1 - Fraction(1, 2 ** 22)))
            hi_ = pins.rne_fp16(exact * (1 + Fraction(1, 2 ** 22)))
            if not (lo_ <= Fraction(float(scale[n, j])) <= hi_) or int(z[n, j]) != 8:
                bad.append((n, j))
    return bad


def test_symmetric_codes_nearest_and_scale():
    """Codes nearest for the stored scale with the fixed zero 8 (brute force over 16 codes),
    scale = fp16(max|w'| / 7); a /8 scale (the other common symmetric form) is caught."""
    W = si.weights(4, 256, offset=115)
    s = np.exp(np.random.default_rng(10).uniform(-1, 1, 256)).astype(np.float16)
    r = oracle.quantize_groups(W, s, zero_point=False)
    w = W.astype(np.float32) * s.astype(np.float32)
    assert not pins.check_codes_nearest(w, r["q"], r["z"], r["scale"])
    assert not _check_symmetric_scale(w, r["z"], r["scale"])
    amax = np.maximum(np.abs(w.reshape(4, 2, 128)).max(axis=2), 2.0 ** -14)
    mutant = (amax / np.float32(8)).astype(np.float16)
    assert _check_symmetric_scale(w, r["z"], mutant)
    # dequantized weights of the signed code: (q - 8) * sc with q - 8 in -8..7
    qz = r["q"].astype(np.int64) - 8
    assert qz.min() >= -8 and qz.max() <= 7


def test_symmetric_search_errors_exact():
    """The scale search with symmetric codes: errors against exact rational arithmetic."""
    X = si.activations(2, 128, offset=116)
    W = si.weights(2, 128, offset=116)
    r = oracle.search_errors(X, W, n_grid=4, zero_point=False)
    for i in range(4):
        qz = oracle.quantize_groups(W, r["s16"][i], zero_point=False)
        exact = pins.exact_search_error(X, W, r["s16"][i], qz["q"], qz["z"], qz["scale"])
        assert abs(r["err"][i] - float(exact)) <= 1e-12 * float(exact)


# ----------------------------------------------------------------- group size 64
@pytest.mark.parametrize("group", [64, 32])
def test_small_group_codes_scales_and_layout(group):
    """64- and 32-channel groups: codes nearest, scale / zero closed form per group, packed
    zeros two groups per byte, byte count; symmetric codes too."""
    W = si.weights(3, 384, offset=117)
    s = np.exp(np.random.default_rng(11).uniform(-1, 1, 384)).astype(np.float16)
    w = W.astype(np.float32) * s.astype(np.float32)
    G = 384 // group
    for zp in (True, False):
        r = oracle.quantize_groups(W, s, zero_point=zp, group=group)
        assert r["scale"].shape == (3, G) and r["z"].shape == (3, G)
        assert not pins.check_codes_nearest(w, r["q"], r["z"], r["scale"])
        if zp:
            assert not pins.check_scale_zero(w, r["z"], r["scale"])
        qw, sc, zb = oracle.pack(r["q"], r["z"], r["scale"])
        assert zb.shape == (3, G // 2)
        q2, z2, s2 = oracle.unpack(qw, sc, zb, 384)
        assert np.array_equal(q2, r["q"]) and np.array_equal(z2, r["z"])
    assert oracle.packed_bytes(4096, 4096, 64) == 4096 * 2048 + 4096 * 64 * 2 + 4096 * 32
    assert oracle.packed_bytes(4096, 4096, 32) == 4096 * 2048 + 4096 * 128 * 2 + 4096 * 64


def test_group32_matches_group64_when_quarters_share_the_range():
    """If each 32-channel quarter of every 64-channel block holds that block's min and max,
    the two group sizes give the same codes and each 64-group's scale and zero twice."""
    rng = np.random.default_rng(13)
    W = (rng.uniform(-0.05, 0.05, (2, 256))).astype(np.float16)
    for b in range(4):
        for half in range(2):
            W[:, b * 64 + half * 32 + 3] = np.float16(-0.06)
            W[:, b * 64 + half * 32 + 30] = np.float16(0.08)
    r64 = oracle.quantize_groups(W, group=64)
    r32 = oracle.quantize_groups(W, group=32)
    assert np.array_equal(r32["q"], r64["q"])
    assert np.array_equal(r32["scale"].view(np.uint16), np.repeat(r64["scale"], 2, axis=1).view(np.uint16))
    assert np.array_equal(r32["z"], np.repeat(r64["z"], 2, axis=1))


def test_group32_search_and_clip_errors_exact():
    X = si.activations(2, 128, offset=119)
    W = si.weights(2, 128, offset=119)
    r = oracle.search_errors(X, W, n_grid=3, group=32)
    for i in range(3):
        qz = oracle.quantize_groups(W, r["s16"][i], group=32)
        exact = pins.exact_search_error(X, W, r["s16"][i], qz["q"], qz["z"], qz["scale"])
        assert abs(r["err"][i] - float(exact)) <= 1e-12 * float(exact)
    e = oracle.clip_errors(X, W, r["s16"][2], 200, 3, group=32)
    assert e.shape == (3, 2, 4)
    qz = oracle.quantize_groups(W, r["s16"][2], np.full((2, 4), oracle.clip_ratios(200, 3)[1], np.float32), group=32)
    ex = pins.exact_group_errors(X, W, r["s16"][2], qz["q"], qz["z"], qz["scale"])
    assert all(abs(e[1, n, g] - float(ex[n][g])) <= 1e-12 * float(ex[n][g]) for n in range(2) for g in range(4))


def test_group64_matches_group128_when_halves_share_the_range():
    """If each 64-channel half of every 128-channel block holds that block's min and max,
    the two group sizes give the same scales (each repeated) and the same codes."""
    rng = np.random.default_rng(12)
    W = (rng.uniform(-0.05, 0.05, (2, 256))).astype(np.float16)
    for b in range(2):
        for half in range(2):
            W[:, b * 128 + half * 64] = np.float16(-0.07)
            W[:, b * 128 + half * 64 + 1] = np.float16(0.09)
    r128 = oracle.quantize_groups(W, group=128)
    r64 = oracle.quantize_groups(W, group=64)
    assert np.array_equal(r64["q"], r128["q"])
    assert np.array_equal(r64["scale"].view(np.uint16), np.repeat(r128["scale"], 2, axis=1).view(np.uint16))
    assert np.array_equal(r64["z"], np.repeat(r128["z"], 2, axis=1))


def test_group64_search_errors_exact():
    X = si.activations(2, 128, offset=118)
    W = si.weights(2, 128, offset=118)
    r = oracle.search_errors(X, W, n_grid=3, group=64)
    for i in range(3):
        qz = oracle.quantize_groups(W, r["s16"][i], group=64)
        exact = pins.exact_search_error(X, W, r["s16"][i], qz["q"], qz["z"], qz["scale"])
        assert abs(r["err"][i] - float(exact)) <= 1e-12 * float(exact)
    e = oracle.clip_errors(X, W, r["s16"][1], 200, 3, group=64)
    qz = oracle.quantize_groups(W, r["s16"][1], np.full((2, 2), oracle.clip_ratios(200, 3)[2], np.float32), group=64)
    ex = pins.exact_group_errors(X, W, r["s16"][1], qz["q"], qz["z"], qz["scale"])
    assert all(abs(e[2, n, g] - float(ex[n][g])) <= 1e-12 * float(ex[n][g]) for n in range(2) for g in range(2))


# ----------------------------------------------------------------- 8-bit codes
@pytest.mark.parametrize("group", [128, 32])
def test_8bit_codes_nearest_scale_and_zero(group):
    """8-bit codes: nearest of 0..255 for the stored scale (brute force), scale / zero from
    the closed form with 255 levels; a 15-level scale is caught by the same check."""
    W = si.weights(3, 256, offset=130)
    s = np.exp(np.random.default_rng(14).uniform(-1, 1, 256)).astype(np.float16)
    w = W.astype(np.float32) * s.astype(np.float32)
    r = oracle.quantize_groups(W, s, group=group, w_bit=8)
    assert not pins.check_codes_nearest(w, r["q"], r["z"], r["scale"], qmax=255)
    assert not pins.check_scale_zero(w, r["z"], r["scale"], qmax=255)
    r4 = oracle.quantize_groups(W, s, group=group, w_bit=4)
    assert pins.check_scale_zero(w, r4["z"], r4["scale"], qmax=255)
    assert r["q"].max() > 15                      # the codes use the wider range


def test_8bit_symmetric_codes():
    """Symmetric 8-bit: sc = max|w'| / 127, zero 128, q - 128 in -128..127, codes nearest."""
    W = si.weights(2, 256, offset=131)
    r = oracle.quantize_groups(W, zero_point=False, w_bit=8)
    w = W.astype(np.float32)
    assert np.all(r["z"] == 128)
    assert not pins.check_codes_nearest(w, r["q"], r["z"], r["scale"], qmax=255)
    for n in range(2):
        for j in range(2):
            amax = np.abs(w[n, j * 128:(j + 1) * 128]).max()
            assert r["scale"][n, j] == np.float16(np.float32(amax) / np.float32(127))
    # the largest magnitude maps to code 128 +- 127
    n, k = np.unravel_index(np.argmax(np.abs(w[:, :128])), (2, 128))
    assert abs(int(r["q"][n, k]) - 128) == 127


def test_8bit_pack_layout_by_hand():
    """Byte j of word w holds channel 4w + j; one zero byte per group; the byte count."""
    q = np.zeros((1, 128), dtype=np.uint8)
    q[0, :8] = [1, 2, 3, 4, 0xA0, 0xB0, 0xC0, 0xD0]
    z = np.array([[0x7F]], dtype=np.uint8)
    sc = np.array([[1.0]], dtype=np.float16)
    qw, scp, zp = oracle.pack(q, z, sc, w_bit=8)
    assert qw.shape == (1, 32) and zp.shape == (1, 1)
    assert qw[0, 0] == 0x04030201 and qw[0, 1] == 0xD0C0B0A0
    assert zp[0, 0] == 0x7F
    q2, z2, s2 = oracle.unpack(qw, scp, zp, 128)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    W = si.weights(5, 384, offset=132)
    r = oracle.quantize_groups(W, group=64, w_bit=8)
    qw, scp, zp = oracle.pack(r["q"], r["z"], r["scale"], w_bit=8)
    q2, z2, _ = oracle.unpack(qw, scp, zp, 384)
    assert np.array_equal(q2, r["q"]) and np.array_equal(z2, r["z"])
    assert oracle.packed_bytes(4096, 4096, 128, w_bit=8) == 4096 * 4096 + 4096 * 32 * 2 + 4096 * 32


def test_8bit_search_and_clip_errors_exact():
    X = si.activations(2, 128, offset=133)
    W = si.weights(2, 128, offset=133)
    r = oracle.search_errors(X, W, n_grid=3, w_bit=8)
    for i in range(3):
        qz = oracle.quantize_groups(W, r["s16"][i], w_bit=8)
        exact = pins.exact_search_error(X, W, r["s16"][i], qz["q"], qz["z"], qz["scale"])
        assert abs(r["err"][i] - float(exact)) <= 1e-12 * float(exact)
    e = oracle.clip_errors(X, W, r["s16"][1], 200, 3, w_bit=8)
    qz = oracle.quantize_groups(W, r["s16"][1], np.full((2, 1), oracle.clip_ratios(200, 3)[2], np.float32), w_bit=8)
    ex = pins.exact_group_errors(X, W, r["s16"][1], qz["q"], qz["z"], qz["scale"])
    assert all(abs(e[2, n, 0] - float(ex[n][0])) <= 1e-12 * float(ex[n][0]) for n in range(2))
    # 8-bit codes quantize more finely: the RTN error falls well below the 4-bit one
    r4 = oracle.search_errors(X, W, n_grid=1)
    assert r["err"][0] < r4["err"][0] / 50


def test_8bit_linear_reference_one_hot():
    """x = e_k reads (q - z) sc of channel k straight from the 8-bit packed words."""
    W = si.weights(3, 256, offset=134)
    qw, sc, zp, _ = oracle.quantize_pack(W, group=64, w_bit=8)
    for k in (0, 5, 63, 64, 255):
        X = np.zeros((1, 256), dtype=np.float16)
        X[0, k] = 1.0
        y, _ = oracle.linear_reference(X, qw, sc, zp, 256)
        for n in range(3):
            code = (int(qw[n, k // 4]) >> (8 * (k % 4))) & 0xFF
            want = (code - int(zp[n, k // 64])) * float(sc[n, k // 64])
            assert y[0, n] == want


# ----------------------------------------------------------------- 3-bit codes
@pytest.mark.parametrize("group", [128, 32])
def test_3bit_codes_nearest_scale_and_zero(group):
    """3-bit codes: nearest of 0..7 for the stored scale (brute force), scale / zero from the
    closed form with 7 levels; the 15-level scale of 4-bit codes fails the same check."""
    W = si.weights(3, 256, offset=140)
    s = np.exp(np.random.default_rng(15).uniform(-1, 1, 256)).astype(np.float16)
    w = W.astype(np.float32) * s.astype(np.float32)
    r = oracle.quantize_groups(W, s, group=group, w_bit=3)
    assert not pins.check_codes_nearest(w, r["q"], r["z"], r["scale"], qmax=7)
    assert not pins.check_scale_zero(w, r["z"], r["scale"], qmax=7)
    r4 = oracle.quantize_groups(W, s, group=group, w_bit=4)
    assert pins.check_scale_zero(w, r4["z"], r4["scale"], qmax=7)
    assert r["q"].max() == 7 and r["q"].min() == 0   # min and max of each group hit the ends


def test_3bit_symmetric_codes():
    """Symmetric 3-bit: sc = max|w'| / 3, zero 4, q - 4 in -4..3, codes nearest."""
    W = si.weights(2, 256, offset=141)
    r = oracle.quantize_groups(W, zero_point=False, w_bit=3)
    w = W.astype(np.float32)
    assert np.all(r["z"] == 4)
    assert not pins.check_codes_nearest(w, r["q"], r["z"], r["scale"], qmax=7)
    for n in range(2):
        for j in range(2):
            amax = np.abs(w[n, j * 128:(j + 1) * 128]).max()
            assert r["scale"][n, j] == np.float16(np.float32(amax) / np.float32(3))
    n, k = np.unravel_index(np.argmax(np.abs(w[:, :128])), (2, 128))
    assert abs(int(r["q"][n, k]) - 4) == 3


def test_3bit_pack_layout_by_hand():
    """Bit planes per 128-channel block: words 0-7 carry bits 0-1 (pair (2f, 2f+1) of word i
    at bits 2f and 16 + 2f), words 8-11 bit 2 (pair p of word 8 + j at bits p and 16 + p);
    zeros in nibbles as for 4-bit; the byte count."""
    q = np.zeros((1, 256), dtype=np.uint8)
    q[0, 0] = 5      # 0b101: word 0 bits 0-1 = 01, word 8 bit 0
    q[0, 1] = 6      # 0b110: word 0 bits 16-17 = 10, word 8 bit 16
    q[0, 17] = 3     # channel 16 + 1: word 1 bits 16-17 = 11
    q[0, 33] = 4     # channel 32 + 1: word 2 bits 16-17 = 00, word 9 bit 16
    q[0, 127] = 7    # channel 112 + 15: word 7 bits 30-31; channel 96 + 31: word 11 bit 31
    q[0, 130] = 1    # block 1, channel 2: word 12 bits 2-3
    z = np.array([[3, 5]], dtype=np.uint8)
    sc = np.array([[1.0, 2.0]], dtype=np.float16)
    qw, scp, zp = oracle.pack(q, z, sc, w_bit=3)
    assert qw.shape == (1, 24) and zp.shape == (1, 1)
    want = [0] * 24
    want[0] = 0x1 | (0x2 << 16)
    want[8] = 0x1 | (0x1 << 16)
    want[1] = 0x3 << 16
    want[9] = 0x1 << 16
    want[7] = 0x3 << 30
    want[11] = 0x1 << 31
    want[12] = 0x1 << 2
    assert [int(v) for v in qw[0]] == want
    assert zp[0, 0] == 0x53
    q2, z2, _ = oracle.unpack(qw, scp, zp, 256)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    W = si.weights(5, 384, offset=142)
    r = oracle.quantize_groups(W, group=32, w_bit=3)
    qw, scp, zp = oracle.pack(r["q"], r["z"], r["scale"], w_bit=3)
    q2, z2, _ = oracle.unpack(qw, scp, zp, 384)
    assert np.array_equal(q2, r["q"]) and np.array_equal(z2, r["z"])
    assert oracle.packed_bytes(4096, 4096, 128, w_bit=3) == 4096 * 1536 + 4096 * 32 * 2 + 4096 * 16


def test_3bit_search_and_clip_errors_exact():
    X = si.activations(2, 128, offset=143)
    W = si.weights(2, 128, offset=143)
    r = oracle.search_errors(X, W, n_grid=3, w_bit=3)
    for i in range(3):
        qz = oracle.quantize_groups(W, r["s16"][i], w_bit=3)
        exact = pins.exact_search_error(X, W, r["s16"][i], qz["q"], qz["z"], qz["scale"])
        assert abs(r["err"][i] - float(exact)) <= 1e-12 * float(exact)
    e = oracle.clip_errors(X, W, r["s16"][1], 200, 3, w_bit=3)
    qz = oracle.quantize_groups(W, r["s16"][1], np.full((2, 1), oracle.clip_ratios(200, 3)[2], np.float32), w_bit=3)
    ex = pins.exact_group_errors(X, W, r["s16"][1], qz["q"], qz["z"], qz["scale"])
    assert all(abs(e[2, n, 0] - float(ex[n][0])) <= 1e-12 * float(ex[n][0]) for n in range(2))
    # 3-bit codes quantize more coarsely: about twice the step, four times the error
    r4 = oracle.search_errors(X, W, n_grid=1)
    assert r["err"][0] > 2 * r4["err"][0]


def test_3bit_linear_reference_one_hot():
    """x = e_k reads (q - z) sc of channel k from the bit planes (bits located by the
    layout's own formula, written out here)."""
    W = si.weights(3, 256, offset=144)
    qw, sc, zp, _ = oracle.quantize_pack(W, group=64, w_bit=3)
    for k in (0, 1, 17, 63, 64, 127, 128, 255):
        X = np.zeros((1, 256), dtype=np.float16)
        X[0, k] = 1.0
        y, _ = oracle.linear_reference(X, qw, sc, zp, 256)
        b, c = divmod(k, 128)
        for n in range(3):
            lo = (int(qw[n, 12 * b + c // 16]) >> (2 * ((c % 16) // 2) + 16 * (c % 2))) & 3
            hi = (int(qw[n, 12 * b + 8 + c // 32]) >> ((c % 32) // 2 + 16 * (c % 2))) & 1
            g = k // 64
            zz = (int(zp[n, g // 2]) >> (4 * (g % 2))) & 0xF
            assert y[0, n] == (lo + 4 * hi - zz) * float(sc[n, g])
