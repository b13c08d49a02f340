"""The no-allocation scale search (awq_search_scales_noalloc, called through the C ABI)
gives the same results as awq_search_scales with a caller-owned workspace, bit for bit,
on two calls in a row, the second with a smaller input (the static array keeps the first
call's contents, which must not leak into the second)."""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from weight_only_bit_02_amd import _abi
from tests.gpu_util import DEV, host, to_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _outs(K, n_grid=20):
    return (torch.empty(K, dtype=torch.float16, device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV),
            torch.empty(n_grid, dtype=torch.float64, device=DEV),
            torch.empty((n_grid, K), dtype=torch.float16, device=DEV))


def _search_both(lib, X, W):
    T, K = X.shape
    N = W.shape[0]
    cfg = _abi.config()
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    # the existing entry point, with its own workspace
    a = _outs(K)
    nbytes = lib.awq_search_workspace_size(T, N, K, C.byref(cfg))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    _abi.check("awq_search_scales", lib.awq_search_scales(
        _p(X), T, _p(W), N, K, C.byref(cfg), _p(a[0]), _p(a[1]), _p(a[2]), _p(a[3]), _p(ws), nbytes,
        None, st))
    # the no-allocation entry point
    b = _outs(K)
    f = torch.zeros(1, dtype=torch.int32, device=DEV)
    _abi.check("awq_search_scales_noalloc", lib.awq_search_scales_noalloc(
        _p(X), T, _p(W), N, K, C.byref(cfg), _p(b[0]), _p(b[1]), _p(b[2]), _p(b[3]), _p(f), st))
    torch.cuda.synchronize()
    return [host(t) for t in a], [host(t) for t in b], int(host(f)[0])


def test_search_noalloc_matches_search_on_two_calls():
    lib = _abi.load()
    for T, N, K, off in ((512, 1024, 4096, 71), (256, 300, 1024, 72)):   # second call smaller
        X = si.activations(T, K, offset=off, channel_offset=K)
        W = si.weights(N, K, offset=off)
        a, b, flags = _search_both(lib, to_dev(X), to_dev(W))
        assert flags == 0
        assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))   # s_best
        assert int(a[1][0]) == int(b[1][0])                                  # best index
        assert np.array_equal(a[2], b[2])                                    # errors, bitwise
        assert np.array_equal(a[3].view(np.uint16), b[3].view(np.uint16))   # candidate scales
        if T == 256:  # the smaller call against the oracle too
            ref = oracle.search_scales(X, W)
            assert np.all(np.abs(b[2] - ref["err"]) <= 1e-5 * ref["err"])
            if ref["gap"] >= 1e-5:
                assert int(b[1][0]) == ref["best_idx"]


def test_search_noalloc_rejects_oversize():
    lib = _abi.load()
    cfg = _abi.config()
    X = torch.zeros((8, 128), dtype=torch.float16, device=DEV)
    o = _outs(28672)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.awq_search_scales_noalloc(_p(X), 8192, _p(X), 4096, 28672, C.byref(cfg), _p(o[0]),
                                         _p(o[1]), None, None, None, st) == 7
