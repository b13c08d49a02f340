"""GPU parity of the weight-clipping search (awq_clip_search) and of the clipped pack
(awq_quantize_pack_clipped) against the oracle.

The chosen ratio index is a floating-point decision: it must equal the oracle's first
minimum wherever the oracle's two smallest errors of that group differ by more than 1e-5
(relative), and the chosen error must match the oracle's to 1e-5 everywhere. Packing with
given indices is integer work and must be bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import DEV, host, packed_host, to_dev

pytestmark = pytest.mark.gpu


def _scales(X, i=8):
    a, _ = oracle.activation_mean_abs(X)
    return oracle.candidate_scales(a, 20)[1][i]


def _check_choice(idx, err_best, ref_err):
    n_shrink = ref_err.shape[0]
    ref_idx = np.argmin(ref_err, axis=0)           # first minimum
    best = np.take_along_axis(ref_err, ref_idx[None], 0)[0]
    srt = np.sort(ref_err, axis=0)
    gap = (srt[1] - srt[0]) / np.maximum(srt[0], 1e-300) if n_shrink > 1 else np.full(best.shape, np.inf)
    decidable = gap > 1e-5
    assert np.array_equal(idx[decidable], ref_idx[decidable])
    assert np.all(np.abs(err_best - best) <= 1e-5 * best + 1e-30)
    return ref_idx


@pytest.mark.parametrize("T,N,K,n_shrink,with_s", [
    (64, 130, 256, 20, True),      # ragged row tile
    (37, 67, 384, 5, False),       # ragged tokens, s = 1
    (512, 128, 1152, 10, True),    # eight waves of tokens, nine groups
    (200, 64, 128, 1, True),       # one-point grid: r = 1
])
def test_clip_search_matches_oracle(T, N, K, n_shrink, with_s):
    X = si.activations(T, K, offset=T + N)
    W = si.weights(N, K, offset=T + N)
    s = _scales(X) if with_s else None
    ref_err = oracle.clip_errors(X, W, s, 200, n_shrink)
    idx, err = awq.clip_search(to_dev(X), to_dev(W), to_dev(s) if with_s else None, 200, n_shrink)
    ref_idx = _check_choice(host(idx).astype(np.int64), host(err), ref_err)
    # packing with the oracle's choice is bit-exact
    ratio = oracle.clip_ratios(200, n_shrink)[ref_idx]
    qw, sc, zb, _ = oracle.quantize_pack(W, s, ratio)
    p = awq.quantize_pack(to_dev(W), to_dev(s) if with_s else None,
                          clip_idx=to_dev(ref_idx.astype(np.uint8)), clip_steps=200)
    gq, gs, gz = packed_host(p)
    assert np.array_equal(gq, qw) and np.array_equal(gz, zb)
    assert np.array_equal(gs.view(np.uint16), sc.view(np.uint16))


def test_clip_lowers_group_errors_end_to_end():
    """Search s, then clip, then pack: every group's chosen error is at most its unclipped
    one, and the layer's calibration output error does not grow."""
    T, N, K = 256, 96, 512
    X = si.activations(T, K, offset=120)
    W = si.weights(N, K, offset=120)
    r = awq.search_scales(to_dev(X), to_dev(W))
    idx, err = awq.clip_search(to_dev(X), to_dev(W), r.s_best, 200, 40)
    ref_err = oracle.clip_errors(X, W, host(r.s_best), 200, 40)
    assert np.all(host(err) <= ref_err[0] * (1 + 1e-5))
    p = awq.quantize_pack(to_dev(W), r.s_best, clip_idx=idx, clip_steps=200)
    Xs = awq.apply_inverse_scale(to_dev(X), r.s_best, 1)
    y = host(awq.linear_w4a16(Xs, p)).astype(np.float64)
    p0 = awq.quantize_pack(to_dev(W), r.s_best)
    y0 = host(awq.linear_w4a16(Xs, p0)).astype(np.float64)
    yt = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.sum((y - yt) ** 2) <= np.sum((y0 - yt) ** 2)


@pytest.mark.slow
def test_clip_7b_o_proj_sampled_rows():
    """Llama-2-7B o_proj (4096 x 4096), 512 calibration tokens, the scale search's s, 20
    ratios; the oracle scores 48 sampled rows (rows are independent)."""
    N, K = si.LLAMA2_7B_SEARCH_GROUPS["o"]
    X = si.activations(512, K, offset=121, channel_offset=K)
    W = si.weights(N, K, offset=121)
    r = awq.search_scales(to_dev(X), to_dev(W))
    s = host(r.s_best)
    idx, err = awq.clip_search(to_dev(X), to_dev(W), r.s_best, 200, 20)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(9).choice(N, 46, replace=False)]))
    ref_err = oracle.clip_errors(X, W[rows], s, 200, 20)
    _check_choice(host(idx)[rows].astype(np.int64), host(err)[rows], ref_err)


# ----------------------------------------------------------------- symmetric codes (f4)
@pytest.mark.parametrize("N,K", [(67, 384), (256, 4096), (130, 11008)])
def test_symmetric_pack_bit_exact_and_linear(N, K):
    W = si.weights(N, K, offset=N + K + 1)
    a, _ = oracle.activation_mean_abs(si.activations(32, K, offset=N))
    s = oracle.candidate_scales(a, 20)[1][6]
    qw, sc, zb, _ = oracle.quantize_pack(W, s, zero_point=False)
    p = awq.quantize_pack(to_dev(W), to_dev(s), zero_point=False)
    gq, gs, gz = packed_host(p)
    assert np.array_equal(gq, qw) and np.array_equal(gz, zb)
    assert np.all(oracle.unpack(qw, sc, zb, K)[1] == 8)   # every group's zero is 8
    assert np.array_equal(gs.view(np.uint16), sc.view(np.uint16))
    for M, kern in ((1, "gemv"), (8, "skinny"), (40, "gemm")):
        X = si.activations(M, K, offset=M + 3)
        Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kern))
        y_ref, bound = oracle.linear_reference(X, qw, sc, zb, K)
        assert oracle.linear_within_tolerance(Y.astype(np.float64), y_ref, bound).all(), kern


@pytest.mark.parametrize("T,N,K", [(96, 192, 512), (512, 130, 1152)])
def test_symmetric_search_and_clip(T, N, K):
    X = si.activations(T, K, offset=T + 5)
    W = si.weights(N, K, offset=T + 5)
    ref = oracle.search_errors(X, W, zero_point=False)
    r = awq.search_scales(to_dev(X), to_dev(W), zero_point=False)
    err = host(r.err)
    assert np.all(np.abs(err - ref["err"]) <= 1e-5 * ref["err"])
    if oracle.relative_gap(ref["err"]) >= 1e-5:
        assert int(host(r.best_idx)[0]) == int(np.argmin(ref["err"]))
    s = host(r.s_best)
    ref_err = oracle.clip_errors(X, W, s, 200, 8, zero_point=False)
    idx, cerr = awq.clip_search(to_dev(X), to_dev(W), r.s_best, 200, 8, zero_point=False)
    ref_idx = _check_choice(host(idx).astype(np.int64), host(cerr), ref_err)
    qw, sc, zb, _ = oracle.quantize_pack(W, s, oracle.clip_ratios(200, 8)[ref_idx], zero_point=False)
    p = awq.quantize_pack(to_dev(W), r.s_best, clip_idx=to_dev(ref_idx.astype(np.uint8)),
                          zero_point=False)
    gq, gs, gz = packed_host(p)
    assert np.array_equal(gq, qw) and np.array_equal(gz, zb)
    assert np.array_equal(gs.view(np.uint16), sc.view(np.uint16))
