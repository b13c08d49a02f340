"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bar: codes, zeros, scales, statistics, candidate scales, chosen grid index and s are
bit-exact; search errors within 1e-5 relative; linear outputs within
|y - y_ref| <= 2e-3 * (|X| |deq W|) per element against the fp64 reference.
Sizes span several tiles plus ragged tails and the degenerate cases.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import DEV, flags_tensor, guarded, guarded_packed, host, packed_host, to_dev

pytestmark = pytest.mark.gpu


def _assert_pack_equal(gpu, ref):
    qw, sc, zb = gpu
    rqw, rsc, rzb = ref[:3]
    assert np.array_equal(qw, rqw), f"codes differ at {np.argwhere(qw != rqw)[:5].tolist()}"
    assert np.array_equal(sc.view(np.uint16), rsc.view(np.uint16)), "scales differ"
    assert np.array_equal(zb, rzb), "zeros differ"


# --------------------------------------------------------------------- quantize + pack
@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (130, 384), (64, 1024), (1024, 1024), (7, 11008)])
def test_quantize_pack_rtn(N, K):
    W = si.weights(N, K, offset=N + K)
    f = flags_tensor()
    out, check = guarded_packed(awq, N, K)
    p = awq.quantize_pack(to_dev(W), flags=f, out=out)
    _assert_pack_equal(packed_host(p), oracle.quantize_pack(W))
    assert int(host(f)[0]) == 0
    check()


@pytest.mark.parametrize("N,K", [(5, 256), (260, 1024)])
def test_quantize_pack_with_scale(N, K):
    W = si.weights(N, K, offset=3 * N)
    a, _ = oracle.activation_mean_abs(si.activations(64, K, offset=N))
    for i in (1, 7, 19):
        s = oracle.candidate_scales(a, 20)[1][i]
        p = awq.quantize_pack(to_dev(W), to_dev(s))
        _assert_pack_equal(packed_host(p), oracle.quantize_pack(W, s))


def test_quantize_pack_degenerate_groups():
    W = si.weights(6, 512, offset=77)
    W[0, :128] = 0.0                              # all-zero group
    W[1, 128:256] = np.float16(0.5)               # constant group
    W[2, 256:384] = np.abs(W[2, 256:384]) + 1     # one-sided group (zero clamps)
    W[3, :] = np.float16(2.0 ** -24)              # subnormal weights
    W[4, 384:512] = np.linspace(-60000, 60000, 128).astype(np.float16)  # widest range
    W[5, 7] = np.float16(65504)
    p = awq.quantize_pack(to_dev(W))
    _assert_pack_equal(packed_host(p), oracle.quantize_pack(W))


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_nonfinite_weight_flags(bad):
    """A NaN or Inf weight raises NONFINITE_INPUT in the pack, the scale search and the
    clip search (a NaN hides from min / max, so the searches also check their errors)."""
    W = si.weights(64, 256, offset=5)
    W[1, 3] = bad
    X = si.activations(64, 256, offset=5)
    f = flags_tensor()
    awq.quantize_pack(to_dev(W), flags=f)
    assert int(host(f)[0]) & oracle.FLAG_NONFINITE_INPUT
    f = flags_tensor()
    awq.search_scales(to_dev(X), to_dev(W), flags=f)
    assert int(host(f)[0]) & oracle.FLAG_NONFINITE_INPUT
    f = flags_tensor()
    awq.clip_search(to_dev(X), to_dev(W), None, 200, 4, flags=f)
    assert int(host(f)[0]) & oracle.FLAG_NONFINITE_INPUT


def test_quantize_pack_flags():
    W = si.weights(2, 256, offset=5)
    W[1, 3] = np.inf
    f = flags_tensor()
    awq.quantize_pack(to_dev(W), flags=f)
    assert int(host(f)[0]) & oracle.FLAG_NONFINITE_INPUT
    W = np.zeros((1, 128), dtype=np.float16)
    W[0, 0], W[0, 1] = -60000.0, 60000.0
    s = np.full(128, 20.0, dtype=np.float16)
    f = flags_tensor()
    p = awq.quantize_pack(to_dev(W), to_dev(s), flags=f)
    assert int(host(f)[0]) == oracle.FLAG_SCALE_CLAMPED
    _assert_pack_equal(packed_host(p), oracle.quantize_pack(W, s))


# --------------------------------------------------------------------- statistic + scales
@pytest.mark.parametrize("T,K", [(1, 128), (37, 384), (256, 1024), (512, 4096), (8192, 256)])
def test_activation_stats_exact(T, K):
    X = si.activations(T, K, offset=T)
    act = host(awq.activation_stats(to_dev(X)))
    ref, _ = oracle.activation_mean_abs(X)
    assert np.array_equal(act, ref)


def test_activation_stats_extremes():
    X = np.full((8192, 128), 65504.0, dtype=np.float16)
    X[::5, 3] = np.float16(-2.0 ** -24)
    act = host(awq.activation_stats(to_dev(X)))
    assert np.array_equal(act, oracle.activation_mean_abs(X)[0])
    X = np.ones((4, 128), dtype=np.float16)
    X[1, 1] = np.nan
    f = flags_tensor()
    awq.activation_stats(to_dev(X), flags=f)
    assert int(host(f)[0]) & oracle.FLAG_NONFINITE_INPUT


@pytest.mark.parametrize("n_grid", [1, 20, 64])
def test_candidate_scales_exact(n_grid):
    g = np.random.default_rng(n_grid)
    a = np.concatenate([np.abs(g.standard_normal(1000)) * 3, [0.0, 2.0 ** -30, 2.0 ** -14, 1.0, 4096.0, 65504.0],
                        g.uniform(0, 40, 18)]).astype(np.float64)[:1024]
    got = host(awq.candidate_scales(to_dev(a), n_grid))
    _, ref16, ref64 = oracle.candidate_scales(a, n_grid)
    hazard = oracle.fp16_midpoint_distance(ref64) < 2.0 ** -40
    same = got.view(np.uint16) == ref16.view(np.uint16)
    assert np.all(same | hazard), np.argwhere(~(same | hazard))[:5]


# --------------------------------------------------------------------- search
def _search_case(T, N, K, off, n_grid=20):
    X = si.activations(T, K, offset=off)
    W = si.weights(N, K, offset=off)
    ref = oracle.search_scales(X, W, n_grid)
    return X, W, ref


@pytest.mark.parametrize("T,N,K", [(256, 1024, 1024), (300, 130, 256), (600, 64, 384), (17, 3, 128),
                                   (512, 192, 1024)])
def test_search_matches_oracle(T, N, K):
    off = T + N
    X, W, ref = _search_case(T, N, K, off)
    if ref["gap"] < 1e-5:
        pytest.skip(f"near tie in the oracle (gap {ref['gap']:.2e}): index parity unpinned for this seed")
    f = flags_tensor()
    r = awq.search_scales(to_dev(X), to_dev(W), flags=f)
    err = host(r.err)
    rel = np.abs(err - ref["err"]) / ref["err"]
    assert np.all(rel <= 1e-5), (rel.max(), err, ref["err"])
    hazard = oracle.fp16_midpoint_distance(ref["s64"]) < 2.0 ** -40
    sg = host(r.s_grid)
    assert np.all((sg.view(np.uint16) == ref["s16"].view(np.uint16)) | hazard)
    assert int(host(r.best_idx)[0]) == ref["best_idx"]
    assert np.array_equal(host(r.s_best).view(np.uint16), ref["s_best"].view(np.uint16))
    assert int(host(f)[0]) == 0
    # the packed result of the chosen scale
    p = awq.quantize_pack(to_dev(W), r.s_best)
    _assert_pack_equal(packed_host(p), (ref["qweight"], ref["scales"], ref["zeros"]))


def test_search_unit_activations_tie_to_first():
    """|x| = 1 -> s = 1 for every grid point -> bitwise equal errors -> index 0."""
    g = np.random.default_rng(9)
    X = np.where(g.integers(0, 2, size=(64, 512)) == 1, 1.0, -1.0).astype(np.float16)
    W = si.weights(96, 512, offset=9)
    r = awq.search_scales(to_dev(X), to_dev(W))
    err = host(r.err)
    assert np.all(err == err[0])
    assert int(host(r.best_idx)[0]) == 0
    ref = oracle.search_errors(X, W)
    assert np.all(np.abs(err - ref["err"]) <= 1e-5 * ref["err"])


def test_search_alpha0_is_rtn_and_deterministic():
    X, W, ref = _search_case(128, 96, 512, 5)
    r1 = awq.search_scales(to_dev(X), to_dev(W))
    r2 = awq.search_scales(to_dev(X), to_dev(W))
    assert np.array_equal(host(r1.err), host(r2.err))
    assert np.all(host(r1.s_grid)[0] == 1.0)
    p0 = awq.quantize_pack(to_dev(W), r1.s_grid[0].contiguous())
    p1 = awq.quantize_pack(to_dev(W))
    for a, b in zip(packed_host(p0), packed_host(p1)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert host(r1.err)[int(host(r1.best_idx)[0])] <= host(r1.err)[0]


# --------------------------------------------------------------------- linear
def _packed_case(N, K, off):
    W = si.weights(N, K, offset=off)
    qw, sc, zb, _ = oracle.quantize_pack(W)
    p = awq.alloc_packed(N, K, DEV)
    p.qweight.copy_(to_dev(qw.view(np.int32)))
    p.scales.copy_(to_dev(sc))
    p.zeros.copy_(to_dev(zb))
    return p, (qw, sc, zb)


def _check_linear(X, p, ref_pack, kernel):
    out, check = guarded((X.shape[0], p.N), torch.float16)
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kernel, out=out))
    check()
    y_ref, bound = oracle.linear_reference(X, *ref_pack, p.K)
    ok = oracle.linear_within_tolerance(Y.astype(np.float64), y_ref, bound)
    assert ok.all(), (np.argwhere(~ok)[:5].tolist(),
                      float(np.max(np.abs(Y - y_ref) / np.maximum(bound, 1e-30))))


@pytest.mark.parametrize("M", list(range(1, 9)))
@pytest.mark.parametrize("N,K", [(1, 128), (67, 384), (256, 4096), (130, 11008)])
def test_gemv_matches_oracle(M, N, K):
    p, ref = _packed_case(N, K, off=N + 3 * K)
    _check_linear(si.activations(M, K, offset=M), p, ref, "gemv")


@pytest.mark.parametrize("M", [1, 2, 3, 7, 8, 9, 16, 17, 31, 32, 33, 47, 64])
@pytest.mark.parametrize("N,K", [(1, 128), (67, 384), (256, 4096), (130, 11008), (33, 1152)])
def test_skinny_matches_oracle(M, N, K):
    """Small-batch MFMA GEMV: every accumulator bucket (M <= 8, 16, 32, and two token tiles
    up to 64), ragged N, K splits that leave some waves without a group (K = 128) or uneven
    (K = 1152)."""
    p, ref = _packed_case(N, K, off=N + 13 * K)
    _check_linear(si.activations(M, K, offset=M + 400), p, ref, "skinny")


@pytest.mark.parametrize("M", [1, 5, 16, 29, 32, 37, 64])
@pytest.mark.parametrize("N,K", [(10301, 256), (12288, 128), (10240, 1152)])
def test_skinny_two_row_tiles_matches_oracle(M, N, K):
    """The skinny kernel's two-row-tile form (a wave multiplies each X piece into two tiles
    of 32 rows; taken from 160 blocks of 64 rows), with ragged rows (10301: 161 blocks, the
    last one 61 rows, its second tile 3 rows past N), the threshold itself (10240) and
    uneven K splits."""
    p, ref = _packed_case(N, K, off=N + 7 * K)
    _check_linear(si.activations(M, K, offset=M + 450), p, ref, "skinny")


@pytest.mark.parametrize("M", [1, 8, 9, 16, 63, 64, 65, 130, 257])
@pytest.mark.parametrize("N,K", [(1, 128), (67, 384), (256, 4096), (130, 1152)])
def test_gemm_matches_oracle(M, N, K):
    p, ref = _packed_case(N, K, off=N + 5 * K)
    _check_linear(si.activations(M, K, offset=M + 100), p, ref, "gemm")


@pytest.mark.parametrize("kernel,M", [("gemv", 1), ("gemv", 4), ("gemm", 32)])
def test_linear_one_hot_exact(kernel, M):
    """x = e_k returns fp16((q - z) sc) bit-exactly: pins nibble order and group indexing."""
    N, K = 96, 512
    p, (qw, sc, zb) = _packed_case(N, K, off=61)
    ks = [0, 7, 8, 127, 128, 300, 511, 64][:M] if M <= 8 else list(range(0, K, K // M))[:M]
    X = np.zeros((M, K), dtype=np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1.0
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kernel))
    y_ref, _ = oracle.linear_reference(X, qw, sc, zb, K)
    assert np.array_equal(Y.view(np.uint16), y_ref.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
def test_linear_zero_input(kernel):
    p, _ = _packed_case(64, 256, off=62)
    Y = host(awq.linear_w4a16(torch.zeros((4, 256), dtype=torch.float16, device=DEV), p, kernel=kernel))
    assert np.all(Y == 0)


def test_linear_auto_dispatch_and_determinism():
    """AUTO picks the vector GEMV up to M = 3, the skinny MFMA GEMV up to 64, the GEMM above
    (each result equals its explicit kernel's bit for bit), deterministically."""
    p, ref = _packed_case(300, 1024, off=63)
    X = si.activations(80, 1024, offset=63)
    assert awq.gemv_max_m() == 64
    for M, kern in ((1, "gemv"), (3, "gemv"), (4, "skinny"), (8, "skinny"), (32, "skinny"),
                    (33, "skinny"), (64, "skinny"), (65, "gemm"), (80, "gemm")):
        Xm = X[:M]
        a = host(awq.linear_w4a16(to_dev(Xm), p))
        b = host(awq.linear_w4a16(to_dev(Xm), p))
        e = host(awq.linear_w4a16(to_dev(Xm), p, kernel=kern))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
        assert np.array_equal(a.view(np.uint16), e.view(np.uint16)), (M, kern)
        y_ref, bound = oracle.linear_reference(Xm, *ref, 1024)
        assert oracle.linear_within_tolerance(a.astype(np.float64), y_ref, bound).all()


@pytest.mark.parametrize("N,K", [
    (4097, 4096), (9000, 1152), (11008, 4096), (4096, 11008),  # one row per wave
    (16389, 4096), (16387, 2048),  # tall: two rows per wave, odd N (last row clamped)
    (129, 18432), (130, 28672),    # 9 and 14 chunks per lane: one batch, one row per wave
    (7, 32768),                    # 16 chunks per lane (the longest row that fits LDS)
    (65, 33024),                   # activation row beyond 64 KiB of LDS: generic kernel
])
def test_gemv_m1_launch_shapes(N, K):
    """Every M = 1 launch shape of the dispatch, ragged row counts included."""
    p, ref = _packed_case(N, K, off=N + K + 7)
    _check_linear(si.activations(1, K, offset=N), p, ref, "gemv")


@pytest.mark.parametrize("kernel,M", [("gemv", 1), ("gemv", 5), ("skinny", 12), ("skinny", 40),
                                      ("gemm", 70), ("auto", 1)])
@pytest.mark.parametrize("where", ["x_nan", "x_inf", "scale_inf", "none"])
def test_linear_flags_nonfinite(kernel, M, where):
    """The linear path reports a NaN or Inf in X or in the group scales in the flags word
    (plain and gated), and leaves it clear for finite data; Y is unchanged by the flag."""
    N, K = 64, 384
    p, ref = _packed_case(N, K, off=64)
    X = si.activations(M, K, offset=65)
    if where == "x_nan":
        X[M - 1, 200] = np.nan
    elif where == "x_inf":
        X[0, 5] = -np.inf
    elif where == "scale_inf":
        p.scales[N - 1, 2] = float("inf")
    for fn in (awq.linear_w4a16, awq.linear_w4a16_gated_silu):
        f = flags_tensor()
        Y = host(fn(to_dev(X), p, kernel=kernel, flags=f))
        Y0 = host(fn(to_dev(X), p, kernel=kernel))
        assert np.array_equal(Y.view(np.uint16), Y0.view(np.uint16))
        assert int(host(f)[0]) == (0 if where == "none" else oracle.FLAG_NONFINITE_INPUT), where


@pytest.mark.parametrize("M", [1, 65, 256, 257, 300])
@pytest.mark.parametrize("N,K", [(1, 128), (67, 384), (256, 4096), (300, 1152)])
def test_gemm_wide_matches_oracle_and_gemm(M, N, K):
    """The 256-row GEMM (128-column tiles at these sizes): ragged M and N (partial tiles on
    both axes), K of 1..32 steps; within the linear tolerance and bit-identical to the 128-row
    GEMM (same channel order, same fp16 widening)."""
    p, ref = _packed_case(N, K, off=N + 9 * K)
    X = si.activations(M, K, offset=M + 700)
    _check_linear(X, p, ref, "gemm_wide")
    a = host(awq.linear_w4a16(to_dev(X), p, kernel="gemm_wide"))
    b = host(awq.linear_w4a16(to_dev(X), p, kernel="gemm"))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("M", [70, 513])
def test_gemm_wide_gated_and_groups(group, M):
    """Gated (fused gate|up, 67 outputs: a partial column tile) and 64-channel groups, against
    the oracle and bit-identical to the 128-row GEMM."""
    nh, K = 67, 1152
    W = si.weights(2 * nh, K, offset=M + group + 1)
    qw, sc, zb, _ = oracle.quantize_pack(W, None, None, True, group, 4)
    p = awq.quantize_pack(to_dev(W), group_size=group)
    X = si.activations(M, K, offset=M + 800)
    out, check = guarded((M, nh), torch.float16)
    H = host(awq.linear_w4a16_gated_silu(to_dev(X), p, kernel="gemm_wide", out=out))
    check()
    h, g, u, bg, bu = oracle.gated_silu_reference(X, qw, sc, zb, K)
    assert oracle.gated_silu_within_tolerance(H.astype(np.float64), g, u, bg, bu).all()
    H1 = host(awq.linear_w4a16_gated_silu(to_dev(X), p, kernel="gemm"))
    assert np.array_equal(H.view(np.uint16), H1.view(np.uint16))
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel="gemm_wide"))
    Y1 = host(awq.linear_w4a16(to_dev(X), p, kernel="gemm"))
    assert np.array_equal(Y.view(np.uint16), Y1.view(np.uint16))
    y_ref, bound = oracle.linear_reference(X, qw, sc, zb, K)
    assert oracle.linear_within_tolerance(Y.astype(np.float64), y_ref, bound).all()


def test_gemm_auto_kernel_choice():
    """AUTO among the two GEMMs: the 256-row GEMM for plain outputs from M = 128 (M = 1024,
    N = 12288 takes its 256-column tiles; M = 2048, N = 12288 and N = 4096 its 128-column
    tiles), for fused gate|up from 160 tiles (gated M = 512, N = 22016: 172); the 128-row GEMM
    below (M = 100; gated M = 256, N = 22016: 86 tiles). Either result equals the explicit
    kernel's bit for bit, and the two GEMMs agree bit for bit."""
    K = 256
    for M, N, gated, wide in ((1024, 12288, False, True), (2048, 12288, False, True),
                              (2048, 4096, False, True), (100, 4096, False, False),
                              (512, 22016, True, True), (256, 22016, True, False)):
        p, ref = _packed_case(N, K, off=N + M + 11)
        X = to_dev(si.activations(M, K, offset=N + M))
        fn = awq.linear_w4a16_gated_silu if gated else awq.linear_w4a16
        a = host(fn(X, p))
        e = host(fn(X, p, kernel="gemm_wide" if wide else "gemm"))
        assert np.array_equal(a.view(np.uint16), e.view(np.uint16)), (M, N, gated)
        o = host(fn(X, p, kernel="gemm" if wide else "gemm_wide"))
        assert np.array_equal(a.view(np.uint16), o.view(np.uint16)), (M, N, gated)
        if not gated:
            rows = np.arange(0, M, 97)
            y_ref, bound = oracle.linear_reference(host(X)[rows], *ref, K)
            assert oracle.linear_within_tolerance(a[rows].astype(np.float64), y_ref, bound).all()


@pytest.mark.parametrize("M,N,group", [(2047, 8191, 128), (1000, 12300, 64)])
def test_gemm_wide_256_column_tiles_ragged(M, N, group):
    """Shapes where the 256-row GEMM keeps 256-column tiles (their whole waves fill the chip
    as well as 128-column tiles would) with a partial last row and column tile, 128- and
    64-channel groups: bit-identical to the 128-row GEMM, sampled rows within the linear
    tolerance of the oracle."""
    K = 128
    W = si.weights(N, K, offset=N + group)
    qw, sc, zb, _ = oracle.quantize_pack(W, None, None, True, group, 4)
    p = awq.quantize_pack(to_dev(W), group_size=group)
    X = to_dev(si.activations(M, K, offset=M + 5))
    a = host(awq.linear_w4a16(X, p, kernel="gemm_wide"))
    b = host(awq.linear_w4a16(X, p, kernel="gemm"))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    rows = np.r_[np.arange(0, M, 131), M - 1]
    y_ref, bound = oracle.linear_reference(host(X)[rows], qw, sc, zb, K)
    assert oracle.linear_within_tolerance(a[rows].astype(np.float64), y_ref, bound).all()


@pytest.mark.parametrize("M,N,K,gated", [(65, 67, 384, False), (300, 300, 1152, False),
                                          (513, 256, 512, False), (257, 134, 1152, True)])
def test_gemm_wide_32_channel_groups(M, N, K, gated):
    """32-channel groups through the 256-row GEMM (two scales and zero nibbles per lane half
    and step): plain and fused gate|up, ragged shapes, bit-identical to the 128-row GEMM and
    within the linear tolerance of the oracle; what AUTO runs from M = 128 (gated: from 160
    tiles, so the 128-row GEMM here)."""
    W = si.weights(N, K, offset=M + N + 5)
    qw, sc, zb, _ = oracle.quantize_pack(W, None, None, True, 32, 4)
    p = awq.quantize_pack(to_dev(W), group_size=32)
    X = si.activations(M, K, offset=M + 29)
    fn = awq.linear_w4a16_gated_silu if gated else awq.linear_w4a16
    out, check = guarded((M, N // 2 if gated else N), torch.float16)
    Y = host(fn(to_dev(X), p, kernel="gemm_wide", out=out))
    check()
    Yg = host(fn(to_dev(X), p, kernel="gemm"))
    assert np.array_equal(Y.view(np.uint16), Yg.view(np.uint16))
    if gated:
        h, g, u, bg, bu = oracle.gated_silu_reference(X, qw, sc, zb, K)
        assert oracle.gated_silu_within_tolerance(Y, g, u, bg, bu).all()
    else:
        y_ref, bound = oracle.linear_reference(X, qw, sc, zb, K)
        assert oracle.linear_within_tolerance(Y.astype(np.float64), y_ref, bound).all()
        if M >= 128:
            Ya = host(awq.linear_w4a16(to_dev(X), p))
            assert np.array_equal(Ya.view(np.uint16), Y.view(np.uint16))

