"""GPU parity of the 64- and 32-channel group formats (group_size = 64, 32) against the oracle.

Every device step that reads or writes groups is covered: quantize + pack (plain,
with s, symmetric, clipped) bit-exact; the scale search and the clip search (errors to
1e-5, decisions wherever the oracle's ranking is decidable); every linear kernel (vector
GEMV in each of its launch shapes, skinny MFMA GEMV, MFMA GEMM, the gated forms) within
the linear tolerance |y - y_ref| <= 2e-3 * (|X| |deq W|). Every test runs for both sizes.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import guarded, host, packed_host, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.parametrize("group", [64, 32])]


def _s(K, offset, i=7):
    a, _ = oracle.activation_mean_abs(si.activations(32, K, offset=offset))
    return oracle.candidate_scales(a, 20)[1][i]


def _pack_both(W, group, s=None, zero_point=True, clip_ratio=None, clip_idx=None):
    qw, sc, zb, _ = oracle.quantize_pack(W, s, clip_ratio, zero_point, group)
    p = awq.quantize_pack(to_dev(W), to_dev(s) if s is not None else None,
                          clip_idx=to_dev(clip_idx) if clip_idx is not None else None,
                          clip_steps=200, zero_point=zero_point, group_size=group)
    return (qw, sc, zb), p


def _assert_same_pack(ref, p):
    qw, sc, zb = ref
    gq, gs, gz = packed_host(p)
    assert gs.shape == sc.shape and gz.shape == zb.shape
    assert np.array_equal(gq, qw)
    assert np.array_equal(gz, zb)
    assert np.array_equal(gs.view(np.uint16), sc.view(np.uint16))


@pytest.mark.parametrize("N,K,with_s,zp", [
    (67, 384, True, True),       # ragged rows, six groups
    (5, 128, False, True),       # the smallest K: two groups, one zero byte
    (256, 4096, True, False),    # symmetric
    (130, 11008, True, True),    # Llama-2-7B down_proj width
])
def test_pack_bit_exact(N, K, with_s, zp, group):
    W = si.weights(N, K, offset=N + K)
    if N > 3:
        W[0, :group] = 0.0                                  # all-zero group
        W[1, group:2 * group] = np.float16(0.5)             # constant group beside a normal one
        W[2, :group] = np.abs(W[2, :group]) + 1             # one-sided group (the zero clamps)
    s = _s(K, N) if with_s else None
    ref, p = _pack_both(W, group, s, zp)
    _assert_same_pack(ref, p)


def _linear_ok(X, ref, p, kernel):
    qw, sc, zb = ref
    K = X.shape[1]
    out, check = guarded((X.shape[0], p.N), torch.float16)
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kernel, out=out)).astype(np.float64)
    check()
    y_ref, bound = oracle.linear_reference(X, qw, sc, zb, K)
    ok = oracle.linear_within_tolerance(Y, y_ref, bound)
    assert ok.all(), (kernel, np.argwhere(~ok)[:4])


@pytest.mark.parametrize("M,N,K,kernel", [
    (1, 96, 384, "gemv"),        # one chunk per lane
    (1, 200, 4096, "gemv"),      # two chunks per lane
    (1, 77, 11008, "gemv"),      # six chunks per lane
    (1, 40, 20480, "gemv"),      # batched single-token kernel
    (1, 24, 40960, "gemv"),      # rows too long to keep X in LDS
    (3, 130, 4096, "gemv"),
    (8, 67, 1152, "gemv"),
    (1, 100, 4096, "skinny"),
    (7, 130, 1152, "skinny"),
    (16, 64, 4096, "skinny"),
    (32, 96, 11008, "skinny"),
    (40, 300, 1152, "gemm"),
    (129, 256, 4096, "gemm"),    # ragged token tile
    (5, 1000, 384, "auto"),
])
def test_linear_kernels(M, N, K, kernel, group):
    W = si.weights(N, K, offset=M + N + K)
    ref, p = _pack_both(W, group, _s(K, M + 1))
    X = si.activations(M, K, offset=M + 5)
    _linear_ok(X, ref, p, kernel)


def test_linear_m1_tall_two_rows_per_wave(group):
    """N >= 16384 with at most two chunks per lane takes the two-rows-per-wave launch;
    the oracle checks a sample of rows (rows are independent)."""
    N, K = 16384, 2048
    W = si.weights(N, K, offset=31)
    ref, p = _pack_both(W, group)
    X = si.activations(1, K, offset=32)
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel="gemv")).astype(np.float64)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(4).choice(N, 254, replace=False)]))
    qw, sc, zb = ref
    y_ref, bound = oracle.linear_reference(X, qw[rows], sc[rows], zb[rows], K)
    assert oracle.linear_within_tolerance(Y[:, rows], y_ref, bound).all()


@pytest.mark.parametrize("M,nh,K,kernel", [
    (1, 96, 4096, "gemv"),
    (1, 40, 20480, "gemv"),
    (4, 67, 1152, "gemv"),
    (12, 80, 4096, "skinny"),
    (70, 130, 1152, "gemm"),
])
def test_gated_kernels(M, nh, K, kernel, group):
    W = si.weights(2 * nh, K, offset=M + nh)
    ref, p = _pack_both(W, group, _s(K, M + 2))
    X = si.activations(M, K, offset=M + 9)
    out, check = guarded((X.shape[0], p.N // 2), torch.float16)
    H = host(awq.linear_w4a16_gated_silu(to_dev(X), p, kernel=kernel, out=out))
    check()
    h, g, u, bg, bu = oracle.gated_silu_reference(X, *ref, K)
    assert oracle.gated_silu_within_tolerance(H, g, u, bg, bu).all(), kernel


def test_dequant_identity_rows(group):
    """x = e_k returns fp16((q - z) sc) of channel k bit-exactly for every output row: pins
    the group index (k // group) and the zero nibble of every group of a 128-channel step."""
    N, K = 40, 512
    W = si.weights(N, K, offset=77)
    ref, p = _pack_both(W, group, _s(K, 78))
    q, z, sc = oracle.unpack(*ref, K)
    ks = [0, 31, 32, 63, 64, 95, 96, 127, 128, 191, 200, 511]
    X = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    want = np.stack([((q[:, k].astype(np.float64) - z[:, k // group]) * sc[:, k // group].astype(np.float64))
                     for k in ks]).astype(np.float16)
    for kernel in ("skinny", "gemm"):
        Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kernel))
        assert np.array_equal(Y.view(np.uint16), want.view(np.uint16)), kernel
    for i0 in range(0, len(ks), 8):   # the vector GEMV takes up to 8 tokens
        Y = host(awq.linear_w4a16(to_dev(X[i0:i0 + 8]), p, kernel="gemv"))
        assert np.array_equal(Y.view(np.uint16), want[i0:i0 + 8].view(np.uint16))
    for i in range(len(ks)):   # one token at a time: the M = 1 kernels
        Y = host(awq.linear_w4a16(to_dev(X[i:i + 1]), p, kernel="gemv"))
        assert np.array_equal(Y.view(np.uint16), want[i:i + 1].view(np.uint16))


@pytest.mark.parametrize("T,N,K,zp", [(96, 192, 512, True), (300, 130, 1152, False)])
def test_search_matches_oracle(T, N, K, zp, group):
    X = si.activations(T, K, offset=T + 11)
    W = si.weights(N, K, offset=T + 11)
    ref = oracle.search_errors(X, W, zero_point=zp, group=group)
    r = awq.search_scales(to_dev(X), to_dev(W), zero_point=zp, group_size=group)
    err = host(r.err)
    assert np.all(np.abs(err - ref["err"]) <= 1e-5 * ref["err"])
    if oracle.relative_gap(ref["err"]) >= 1e-5:
        assert int(host(r.best_idx)[0]) == int(np.argmin(ref["err"]))


def _check_choice(idx, err_best, ref_err):
    ref_idx = np.argmin(ref_err, axis=0)
    best = np.take_along_axis(ref_err, ref_idx[None], 0)[0]
    srt = np.sort(ref_err, axis=0)
    gap = (srt[1] - srt[0]) / np.maximum(srt[0], 1e-300) if ref_err.shape[0] > 1 else np.inf
    decidable = gap > 1e-5
    assert np.array_equal(idx[decidable], ref_idx[decidable])
    assert np.all(np.abs(err_best - best) <= 1e-5 * best + 1e-30)
    return ref_idx


@pytest.mark.parametrize("T,N,K,n_shrink,with_s,zp", [
    (64, 130, 256, 20, True, True),     # ragged row tile
    (37, 67, 384, 5, False, True),      # ragged tokens
    (512, 128, 1152, 10, True, False),  # eight waves of tokens, symmetric
    (300, 96, 512, 7, True, True),      # eight waves, the last three without tokens
])
def test_clip_search_and_clipped_pack(T, N, K, n_shrink, with_s, zp, group):
    X = si.activations(T, K, offset=T + N + 1)
    W = si.weights(N, K, offset=T + N + 1)
    s = _s(K, T) if with_s else None
    ref_err = oracle.clip_errors(X, W, s, 200, n_shrink, zp, group)
    assert ref_err.shape == (n_shrink, N, K // group)
    idx, err = awq.clip_search(to_dev(X), to_dev(W), to_dev(s) if with_s else None, 200, n_shrink,
                               zero_point=zp, group_size=group)
    ref_idx = _check_choice(host(idx).astype(np.int64), host(err), ref_err)
    ratio = oracle.clip_ratios(200, n_shrink)[ref_idx]
    ref, p = _pack_both(W, group, s, zp, clip_ratio=ratio, clip_idx=ref_idx.astype(np.uint8))
    _assert_same_pack(ref, p)
