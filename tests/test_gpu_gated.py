"""GPU parity of the fused gate|up MLP module (awq_linear_w4a16_gated_silu) against the
oracle: h = SiLU(x W_gate^T) * (x W_up^T) over one packed weight, gate rows first.

Every GEMV launch shape (single batch, batched, activation row beyond LDS) and the
MFMA GEMM with ragged tiles are covered; at the Llama-2-7B gate|up shape the outputs
are checked on sampled columns, whose gate and up rows the oracle takes one by one.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import DEV, guarded, host, packed_host, to_dev

pytestmark = pytest.mark.gpu


def _gated_case(nh, K, off):
    W = si.weights(2 * nh, K, offset=off)
    qw, sc, zb, _ = oracle.quantize_pack(W)
    p = awq.alloc_packed(2 * nh, K, DEV)
    p.qweight.copy_(to_dev(qw.view(np.int32)))
    p.scales.copy_(to_dev(sc))
    p.zeros.copy_(to_dev(zb))
    return p, (qw, sc, zb)


def _check(X, p, ref, kernel):
    out, check = guarded((X.shape[0], p.N // 2), torch.float16)
    H = host(awq.linear_w4a16_gated_silu(to_dev(X), p, kernel=kernel, out=out))
    check()
    h, g, u, bg, bu = oracle.gated_silu_reference(X, *ref, p.K)
    assert H.shape == h.shape
    ok = oracle.gated_silu_within_tolerance(H.astype(np.float64), g, u, bg, bu)
    assert ok.all(), (np.argwhere(~ok)[:5].tolist(), H[~ok][:5], h[~ok][:5])


@pytest.mark.parametrize("M", list(range(1, 9)))
@pytest.mark.parametrize("nh,K", [(1, 128), (67, 384), (128, 4096), (65, 11008)])
def test_gated_gemv_matches_oracle(M, nh, K):
    p, ref = _gated_case(nh, K, off=nh + 7 * K)
    _check(si.activations(M, K, offset=M + 200), p, ref, "gemv")


@pytest.mark.parametrize("nh,K", [(33, 18432), (9, 33024), (8195, 4096)])
def test_gated_gemv_long_rows_and_tall(nh, K):
    """Batched kernel (more than 8 chunks per lane), the generic kernel (activation row
    beyond 64 KiB of LDS) and an odd number of outputs on the single-batch kernel."""
    p, ref = _gated_case(nh, K, off=nh + K)
    _check(si.activations(1, K, offset=nh), p, ref, "gemv")


@pytest.mark.parametrize("M", [1, 5, 8, 16, 17, 32, 33, 47, 64])
@pytest.mark.parametrize("nh,K", [(1, 128), (67, 384), (200, 1152), (40, 11008)])
def test_gated_skinny_matches_oracle(M, nh, K):
    """Every accumulator bucket of the skinny kernel, the two-token-tile form (M = 33..64)
    included, with ragged outputs."""
    p, ref = _gated_case(nh, K, off=nh + 17 * K)
    _check(si.activations(M, K, offset=M + 500), p, ref, "skinny")


@pytest.mark.parametrize("M", [2, 16, 30, 33, 64])
@pytest.mark.parametrize("nh,K", [(16400, 128), (16384, 384)])
def test_gated_skinny_two_row_tiles(M, nh, K):
    """The gated skinny kernel's two-row-tile form (taken from 512 blocks of 32 outputs),
    ragged (16400 outputs: 513 blocks, the last one's second tile wholly past the end) and
    even (16384: exactly the threshold)."""
    p, ref = _gated_case(nh, K, off=nh + 29 * K)
    _check(si.activations(M, K, offset=M + 520), p, ref, "skinny")


@pytest.mark.parametrize("M", [33, 47, 64])
@pytest.mark.parametrize("group", [64, 32])
def test_gated_skinny_two_tiles_small_groups(M, group):
    """The two-token-tile gated skinny kernel with 64- and 32-channel groups (ragged
    outputs: 67 gate|up pairs)."""
    nh, K = 67, 1152
    W = si.weights(2 * nh, K, offset=M + group)
    qw, sc, zb, _ = oracle.quantize_pack(W, None, None, True, group, 4)
    p = awq.quantize_pack(to_dev(W), group_size=group)
    gq, gs, gz = packed_host(p)
    assert np.array_equal(gq, qw) and np.array_equal(gz, zb)
    assert np.array_equal(gs.view(np.uint16), sc.view(np.uint16))
    X = si.activations(M, K, offset=M + 600)
    H = host(awq.linear_w4a16_gated_silu(to_dev(X), p, kernel="skinny"))
    h, g, u, bg, bu = oracle.gated_silu_reference(X, qw, sc, zb, K)
    assert oracle.gated_silu_within_tolerance(H.astype(np.float64), g, u, bg, bu).all()


@pytest.mark.parametrize("M", [1, 9, 64, 130, 257])
@pytest.mark.parametrize("nh,K", [(1, 128), (67, 384), (200, 1152)])
def test_gated_gemm_matches_oracle(M, nh, K):
    p, ref = _gated_case(nh, K, off=nh + 11 * K)
    _check(si.activations(M, K, offset=M + 300), p, ref, "gemm")


def test_gated_zero_input_and_determinism():
    p, ref = _gated_case(64, 512, off=93)
    Z = host(awq.linear_w4a16_gated_silu(torch.zeros((3, 512), dtype=torch.float16, device=DEV), p))
    assert np.all(Z == 0)
    X = to_dev(si.activations(16, 512, offset=93))
    for kernel in ("gemv", "gemm"):
        Xk = X[:8] if kernel == "gemv" else X
        a = host(awq.linear_w4a16_gated_silu(Xk, p, kernel=kernel))
        b = host(awq.linear_w4a16_gated_silu(Xk, p, kernel=kernel))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 64, 2048])
def test_gated_7b_gate_up_sampled(M):
    """Llama-2-7B gate|up (2 x 11008 rows, K = 4096) under the automatic kernel choice: the
    benchmark's fused decode launch (M = 1), the two-token-tile skinny kernel (M = 64) and
    the GEMM (M = 2048)."""
    nh, K = 11008, 4096
    W = si.weights(2 * nh, K, offset=94)
    p = awq.quantize_pack(to_dev(W))
    X = si.activations(M, K, offset=94, channel_offset=K)
    H = host(awq.linear_w4a16_gated_silu(to_dev(X), p))
    cols = np.unique(np.concatenate([[0, nh - 1], np.random.default_rng(M).choice(nh, 96, replace=False)]))
    qw, sc, zb = packed_host(p)
    rows = np.concatenate([cols, nh + cols])
    ref = oracle.quantize_pack(W[rows])[:3]      # the oracle packs the sampled rows itself
    assert np.array_equal(qw[rows], ref[0]) and np.array_equal(zb[rows], ref[2])
    assert np.array_equal(sc[rows].view(np.uint16), ref[1].view(np.uint16))
    h, g, u, bg, bu = oracle.gated_silu_reference(X, *ref, K)
    ok = oracle.gated_silu_within_tolerance(H[:, cols].astype(np.float64), g, u, bg, bu)
    assert ok.all(), np.argwhere(~ok)[:5]
