"""GPU parity of the 8-bit code format (w_bit = 8) against the oracle.

Quantize + pack (plain, with s, symmetric, clipped) bit-exact; the scale search and the
clip search (errors to 1e-5, decisions wherever the oracle's ranking is decidable).
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import flags_tensor, guarded, host, packed_host, to_dev

pytestmark = pytest.mark.gpu


def _s(K, offset, i=7):
    a, _ = oracle.activation_mean_abs(si.activations(32, K, offset=offset))
    return oracle.candidate_scales(a, 20)[1][i]


def _pack_both(W, group, s=None, zero_point=True, clip_ratio=None, clip_idx=None):
    qw, sc, zb, _ = oracle.quantize_pack(W, s, clip_ratio, zero_point, group, w_bit=8)
    p = awq.quantize_pack(to_dev(W), to_dev(s) if s is not None else None,
                          clip_idx=to_dev(clip_idx) if clip_idx is not None else None,
                          clip_steps=200, zero_point=zero_point, group_size=group, w_bit=8)
    return (qw, sc, zb), p


def _assert_same_pack(ref, p):
    qw, sc, zb = ref
    gq, gs, gz = packed_host(p)
    assert gq.shape == qw.shape and gs.shape == sc.shape and gz.shape == zb.shape
    assert np.array_equal(gq, qw)
    assert np.array_equal(gz, zb)
    assert np.array_equal(gs.view(np.uint16), sc.view(np.uint16))


@pytest.mark.parametrize("N,K,group,with_s,zp", [
    (67, 384, 128, True, True),
    (5, 128, 64, False, True),
    (256, 4096, 128, True, False),     # symmetric
    (130, 11008, 32, True, True),
])
def test_pack_bit_exact(N, K, group, with_s, zp):
    W = si.weights(N, K, offset=N + K + 8)
    if N > 3:
        W[0, :group] = 0.0
        W[1, group:2 * group] = np.float16(0.5)
        W[2, :group] = np.abs(W[2, :group]) + 1
    s = _s(K, N) if with_s else None
    ref, p = _pack_both(W, group, s, zp)
    _assert_same_pack(ref, p)


def test_pack_flags():
    W = si.weights(4, 256, offset=81)
    W[1, 3] = np.nan
    f = flags_tensor()
    awq.quantize_pack(to_dev(W), flags=f, w_bit=8)
    assert int(host(f)[0]) & oracle.FLAG_NONFINITE_INPUT


@pytest.mark.parametrize("T,N,K,zp,group", [(96, 192, 512, True, 128), (300, 130, 1152, False, 64)])
def test_search_matches_oracle(T, N, K, zp, group):
    X = si.activations(T, K, offset=T + 21)
    W = si.weights(N, K, offset=T + 21)
    ref = oracle.search_errors(X, W, zero_point=zp, group=group, w_bit=8)
    r = awq.search_scales(to_dev(X), to_dev(W), zero_point=zp, group_size=group, w_bit=8)
    err = host(r.err)
    assert np.all(np.abs(err - ref["err"]) <= 1e-5 * ref["err"])
    if oracle.relative_gap(ref["err"]) >= 1e-5:
        assert int(host(r.best_idx)[0]) == int(np.argmin(ref["err"]))


@pytest.mark.parametrize("T,N,K,n_shrink,group", [(64, 130, 256, 20, 128), (512, 128, 1152, 10, 32)])
def test_clip_search_and_clipped_pack(T, N, K, n_shrink, group):
    X = si.activations(T, K, offset=T + N + 2)
    W = si.weights(N, K, offset=T + N + 2)
    s = _s(K, T)
    ref_err = oracle.clip_errors(X, W, s, 200, n_shrink, True, group, w_bit=8)
    idx, err = awq.clip_search(to_dev(X), to_dev(W), to_dev(s), 200, n_shrink, group_size=group, w_bit=8)
    ref_idx = np.argmin(ref_err, axis=0)
    best = np.take_along_axis(ref_err, ref_idx[None], 0)[0]
    srt = np.sort(ref_err, axis=0)
    decidable = (srt[1] - srt[0]) / np.maximum(srt[0], 1e-300) > 1e-5
    assert np.array_equal(host(idx).astype(np.int64)[decidable], ref_idx[decidable])
    assert np.all(np.abs(host(err) - best) <= 1e-5 * best + 1e-30)
    ratio = oracle.clip_ratios(200, n_shrink)[ref_idx]
    ref, p = _pack_both(W, group, s, True, clip_ratio=ratio, clip_idx=ref_idx.astype(np.uint8))
    _assert_same_pack(ref, p)


# ----------------------------------------------------------------- linear kernels
@pytest.mark.parametrize("M,N,K,kernel,group", [
    (1, 96, 384, "gemv", 128),
    (1, 200, 4096, "gemv", 64),
    (1, 77, 11008, "gemv", 32),
    (3, 130, 4096, "gemv", 128),
    (8, 67, 1152, "gemv", 64),
    (1, 100, 4096, "skinny", 128),
    (7, 130, 1152, "skinny", 64),
    (16, 64, 4096, "skinny", 32),
    (32, 96, 11008, "skinny", 128),
    (33, 130, 1152, "skinny", 64),
    (64, 67, 4096, "skinny", 32),
    (50, 96, 11008, "skinny", 128),
    (40, 300, 1152, "gemm", 128),
    (129, 256, 4096, "gemm", 64),
    (70, 96, 1152, "gemm", 32),
    (5, 1000, 384, "auto", 128),
    (20, 300, 512, "auto", 128),
    (50, 300, 512, "auto", 128),
    (70, 300, 512, "auto", 128),
])
def test_linear_kernels(M, N, K, kernel, group):
    W = si.weights(N, K, offset=M + N + K + 8)
    ref, p = _pack_both(W, group, _s(K, M + 1))
    X = si.activations(M, K, offset=M + 6)
    out, check = guarded((X.shape[0], p.N), torch.float16)
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kernel, out=out)).astype(np.float64)
    check()
    y_ref, bound = oracle.linear_reference(X, *ref, K)
    ok = oracle.linear_within_tolerance(Y, y_ref, bound)
    assert ok.all(), (kernel, np.argwhere(~ok)[:4])


@pytest.mark.parametrize("M,nh,K,kernel,group", [
    (1, 96, 4096, "gemv", 128),
    (4, 67, 1152, "gemv", 32),
    (12, 80, 4096, "skinny", 64),
    (40, 67, 1152, "skinny", 128),
    (70, 130, 1152, "gemm", 128),
    (40, 64, 512, "gemm", 32),
])
def test_gated_kernels(M, nh, K, kernel, group):
    W = si.weights(2 * nh, K, offset=M + nh + 8)
    ref, p = _pack_both(W, group, _s(K, M + 2))
    X = si.activations(M, K, offset=M + 10)
    out, check = guarded((X.shape[0], p.N // 2), torch.float16)
    H = host(awq.linear_w4a16_gated_silu(to_dev(X), p, kernel=kernel, out=out))
    check()
    h, g, u, bg, bu = oracle.gated_silu_reference(X, *ref, K)
    assert oracle.gated_silu_within_tolerance(H, g, u, bg, bu).all(), kernel


@pytest.mark.parametrize("group", [128, 64, 32])
def test_dequant_identity_rows(group):
    """x = e_k returns fp16((q - z) sc) of channel k bit-exactly through every kernel: pins the
    byte order, the group index and the zero byte of every group of a 128-channel step."""
    N, K = 40, 512
    W = si.weights(N, K, offset=79)
    ref, p = _pack_both(W, group, _s(K, 80), zero_point=group != 64)
    q, z, sc = oracle.unpack(*ref, K)
    ks = [0, 1, 2, 3, 4, 31, 32, 63, 64, 95, 96, 127, 128, 200, 511]
    X = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    want = np.stack([((q[:, k].astype(np.float64) - z[:, k // group]) * sc[:, k // group].astype(np.float64))
                     for k in ks]).astype(np.float16)
    for kernel in ("skinny", "gemm", "gemm_wide"):
        Y = host(awq.linear_w4a16(to_dev(X), p, kernel=kernel))
        assert np.array_equal(Y.view(np.uint16), want.view(np.uint16)), kernel
    for i0 in range(0, len(ks), 8):
        Y = host(awq.linear_w4a16(to_dev(X[i0:i0 + 8]), p, kernel="gemv"))
        assert np.array_equal(Y.view(np.uint16), want[i0:i0 + 8].view(np.uint16))


@pytest.mark.parametrize("M,N,K,group,zp", [
    (65, 67, 384, 128, True),
    (256, 300, 1152, 64, True),
    (257, 256, 4096, 128, False),
    (300, 1, 128, 128, True),
    (1000, 1000, 512, 64, False),
    (129, 200, 1152, 32, True),
    (512, 256, 512, 32, False),
])
def test_gemm_wide_8bit(M, N, K, group, zp):
    """The 256-row GEMM on 8-bit codes (128-column tiles): ragged M and N, 1 to 32 steps, 128-,
    64- and 32-channel groups, with and without the zero point; bit-identical to the 128-row GEMM (same
    widening, same MFMA sequence per output), within the linear tolerance of the oracle, and
    what AUTO runs from M = 128."""
    W = si.weights(N, K, offset=M + N + K + 31)
    ref, p = _pack_both(W, group, _s(K, M + 3), zero_point=zp)
    X = si.activations(M, K, offset=M + 17)
    out, check = guarded((M, N), torch.float16)
    Y = host(awq.linear_w4a16(to_dev(X), p, kernel="gemm_wide", out=out))
    check()
    Yg = host(awq.linear_w4a16(to_dev(X), p, kernel="gemm"))
    assert np.array_equal(Y.view(np.uint16), Yg.view(np.uint16))
    rows = np.r_[np.arange(0, M, 7), M - 1]
    y_ref, bound = oracle.linear_reference(X[rows], *ref, K)
    ok = oracle.linear_within_tolerance(Y[rows].astype(np.float64), y_ref, bound)
    assert ok.all(), np.argwhere(~ok)[:4]
    if M >= 128:
        Ya = host(awq.linear_w4a16(to_dev(X), p))
        assert np.array_equal(Ya.view(np.uint16), Y.view(np.uint16))


def test_gemm_wide_8bit_auto_threshold_and_gated():
    """AUTO keeps the 128-row GEMM below M = 128; the gated epilogue on 8-bit codes stays on the
    128-row GEMM (an explicit wide request is refused)."""
    N, K = 256, 512
    W = si.weights(N, K, offset=91)
    ref, p = _pack_both(W, 128, _s(K, 92))
    X = to_dev(si.activations(100, K, offset=93))
    a = host(awq.linear_w4a16(X, p))
    e = host(awq.linear_w4a16(X, p, kernel="gemm"))
    assert np.array_equal(a.view(np.uint16), e.view(np.uint16))
    with pytest.raises(awq.AwqError):
        awq.linear_w4a16_gated_silu(X, p, kernel="gemm_wide")
