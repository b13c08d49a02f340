"""GPU parity at the full Llama-2-7B / 70B sizes, in the launch configuration the benchmark
times (same entry points, same shapes, device-resident inputs).

Where the oracle can finish the whole problem in a minute or two it does (the full
20-point search of every shared-input group); elsewhere it checks sampled outputs it
computes one by one (rows of a packed matrix, elements of Y).
"""

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import DEV, host, packed_host, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

GROUPS_7B = si.LLAMA2_7B_SEARCH_GROUPS
CALIB_T = 512


@functools.lru_cache(maxsize=4)
def _weights(N, K, offset):
    W = si.weights(N, K, offset=offset)
    W.setflags(write=False)
    return W


def _rows_sample(N, n=192, seed=0):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], g.choice(N, size=n, replace=False)]))


@pytest.mark.parametrize("group", list(GROUPS_7B))
def test_quantize_pack_7b_group(group):
    N, K = GROUPS_7B[group]
    W = _weights(N, K, 7)
    a, _ = oracle.activation_mean_abs(si.activations(64, K, offset=3))
    s = oracle.candidate_scales(a, 20)[1][9]
    p = awq.quantize_pack(to_dev(W), to_dev(s))
    qw, sc, zb = packed_host(p)
    rows = _rows_sample(N, 512)
    rqw, rsc, rzb, _ = oracle.quantize_pack(W[rows], s)
    assert np.array_equal(qw[rows], rqw)
    assert np.array_equal(sc[rows].view(np.uint16), rsc.view(np.uint16))
    assert np.array_equal(zb[rows], rzb)


@pytest.mark.parametrize("group", list(GROUPS_7B))
def test_search_7b_group_full(group):
    """The full 20-point search of each 7B shared-input group (T = 512), the benchmark's
    searches, against the oracle: all 20 errors, the first-minimum index, every candidate
    scale and the chosen one (q|k|v and gate|up take the oracle about a minute each)."""
    N, K = GROUPS_7B[group]
    off = {"qkv": 42, "o": 40, "gate_up": 44, "down": 46}[group]
    X = si.activations(CALIB_T, K, offset=off, channel_offset=K)
    W = si.weights(N, K, offset=off + 1)
    r = awq.search_scales(to_dev(X), to_dev(W))
    err, best = host(r.err), int(host(r.best_idx)[0])
    ref = oracle.search_errors(X, W)
    rel = np.abs(err - ref["err"]) / ref["err"]
    assert np.all(rel <= 1e-5), (rel.max(), int(rel.argmax()))
    hazard = oracle.fp16_midpoint_distance(ref["s64"]) < 2.0 ** -40
    assert np.all((host(r.s_grid).view(np.uint16) == ref["s16"].view(np.uint16)) | hazard)
    ref_best = 0
    for i in range(1, len(ref["err"])):    # the oracle's first minimum
        if ref["err"][i] < ref["err"][ref_best]:
            ref_best = i
    if oracle.relative_gap(ref["err"]) < 1e-5:
        pytest.skip(f"near tie in the oracle: index parity unpinned for {group}")
    assert best == ref_best, (best, ref_best)
    assert np.array_equal(host(r.s_best).view(np.uint16), ref["s16"][ref_best].view(np.uint16))


def _check_sampled_linear(X, p, W_rows_ref, rows, Y):
    """Y[:, rows] against the fp64 reference of those packed rows."""
    qw, sc, zb = W_rows_ref
    y_ref, bound = oracle.linear_reference(X, qw, sc, zb, p.K)
    ok = oracle.linear_within_tolerance(Y[:, rows].astype(np.float64), y_ref, bound)
    assert ok.all(), np.argwhere(~ok)[:5]


@pytest.mark.parametrize("M", [1, 8, 16, 64, 2048])
@pytest.mark.parametrize("group", list(GROUPS_7B))
def test_linear_7b_group(group, M):
    N, K = GROUPS_7B[group]
    W = _weights(N, K, 7)
    p = awq.quantize_pack(to_dev(W))
    X = si.activations(M, K, offset=M, channel_offset=K)
    Y = host(awq.linear_w4a16(to_dev(X), p))
    rows = _rows_sample(N, 96 if M >= 64 else 256, seed=M)
    ref = oracle.quantize_pack(W[rows])[:3]      # the oracle packs the sampled rows itself
    qw, sc, zb = packed_host(p)
    assert np.array_equal(qw[rows], ref[0]) and np.array_equal(zb[rows], ref[2])
    assert np.array_equal(sc[rows].view(np.uint16), ref[1].view(np.uint16))
    _check_sampled_linear(X, p, ref, rows, Y)


# ----------------------------------------------------------------- format variants
# Each variant as the benchmark times it (every variant packs the same weights with one
# config field changed): pack bit-exact on sampled rows, and the decode (M = 1: fused
# gate|up, down) and prefill (M = 2048: q|k|v) outputs of those rows against the oracle.
VARIANTS = {"group64": {"group_size": 64}, "group32": {"group_size": 32},
            "symmetric": {"zero_point": False}, "int8": {"w_bit": 8}, "int3": {"w_bit": 3}}


@pytest.mark.parametrize("gname,M", [("gate_up", 1), ("down", 1), ("qkv", 2048)])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_variant_7b_pack_and_linear(variant, gname, M):
    kw = VARIANTS[variant]
    group, w_bit, zp = kw.get("group_size", 128), kw.get("w_bit", 4), kw.get("zero_point", True)
    N, K = GROUPS_7B[gname]
    W = _weights(N, K, 7)
    a, _ = oracle.activation_mean_abs(si.activations(64, K, offset=3))
    s = oracle.candidate_scales(a, 20)[1][9]
    p = awq.quantize_pack(to_dev(W), to_dev(s), zero_point=zp, group_size=group, w_bit=w_bit)
    X = si.activations(M, K, offset=M + 1, channel_offset=K)
    qw, sc, zb = packed_host(p)
    if gname == "gate_up":  # fused module: output j reads gate row j and up row j + N/2
        nh = N // 2
        outs = _rows_sample(nh, 96, seed=5)
        rows = np.concatenate([outs, outs + nh])
    else:
        outs = rows = _rows_sample(N, 64 if M > 1 else 128, seed=6)
    ref = oracle.quantize_pack(W[rows], s, None, zp, group, w_bit)[:3]
    assert np.array_equal(qw[rows], ref[0]) and np.array_equal(zb[rows], ref[2])
    assert np.array_equal(sc[rows].view(np.uint16), ref[1].view(np.uint16))
    if gname == "gate_up":
        H = host(awq.linear_w4a16_gated_silu(to_dev(X), p))
        h, g, u, bg, bu = oracle.gated_silu_reference(X, *ref, K)
        assert oracle.gated_silu_within_tolerance(H[:, outs], g, u, bg, bu).all()
    else:
        Y = host(awq.linear_w4a16(to_dev(X), p))
        _check_sampled_linear(X, p, ref, rows, Y)


def test_linear_7b_per_matrix_row_slices():
    """Row slices of a group's packed tensor are the packed per-matrix weights."""
    N, K = GROUPS_7B["qkv"]
    W = si.weights(N, K, offset=8)
    p = awq.quantize_pack(to_dev(W))
    x = si.activations(1, K, offset=8, channel_offset=K)
    yf = host(awq.linear_w4a16(to_dev(x), p))
    for off in (0, 4096, 8192):
        v = awq.PackedLinear(p.qweight[off:off + 4096], p.scales[off:off + 4096], p.zeros[off:off + 4096], 4096, K)
        ym = host(awq.linear_w4a16(to_dev(x), v))
        assert np.array_equal(ym.view(np.uint16), yf[:, off:off + 4096].view(np.uint16))


@pytest.mark.parametrize("name", ["qkv_proj", "down_proj"])
def test_70b_layer_pack_and_linear(name):
    """Llama-2-70B shapes: packed rows exact, GEMV (M = 1) and GEMM (M = 32) sampled."""
    N, K = si.LLAMA2_70B_LINEARS[name]
    W = si.weights(N, K, offset=70)
    p = awq.quantize_pack(to_dev(W))
    qw, sc, zb = packed_host(p)
    rows = _rows_sample(N, 128, seed=70)
    rqw, rsc, rzb, _ = oracle.quantize_pack(W[rows])
    assert np.array_equal(qw[rows], rqw) and np.array_equal(zb[rows], rzb)
    assert np.array_equal(sc[rows].view(np.uint16), rsc.view(np.uint16))
    assert p.nbytes() == oracle.packed_bytes(N, K)
    for M in (1, 32):
        X = si.activations(M, K, offset=M, channel_offset=K)
        Y = host(awq.linear_w4a16(to_dev(X), p))
        _check_sampled_linear(X, p, (rqw, rsc, rzb), rows, Y)
    del p
    torch.cuda.empty_cache()
