"""GPU parity of the scale search where the candidate scales span many octaves.

A few channels carry far larger activations than the rest ("AWQ量化实战" §1.3), so
s = mean|x|^alpha can range over several orders of magnitude within one layer, and
the error terms D = W - Q(W diag(s)) diag(1/s) then do too (D of a small-s channel is
the step of its group divided by s). The grid search scores every alpha on the
output error ("AWQ量化实战" §2.2, §3.3 step 4), so its errors, chosen index and scale
must still match the oracle here: errors within 1e-5 relative, index and scales
bit-exact (unless the oracle's two smallest errors are within 1e-5).
"""

import numpy as np
import pytest

import oracle
import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import flags_tensor, host, packed_host, to_dev

pytestmark = pytest.mark.gpu


def _check_search(X, W):
    ref = oracle.search_scales(X, W)
    f = flags_tensor()
    r = awq.search_scales(to_dev(X), to_dev(W), flags=f)
    err = host(r.err)
    rel = np.abs(err - ref["err"]) / ref["err"]
    assert np.all(rel <= 1e-5), (rel.max(), int(rel.argmax()))
    hazard = oracle.fp16_midpoint_distance(ref["s64"]) < 2.0 ** -40
    assert np.all((host(r.s_grid).view(np.uint16) == ref["s16"].view(np.uint16)) | hazard)
    assert int(host(f)[0]) == 0
    if ref["gap"] < 1e-5:
        pytest.skip(f"near tie in the oracle (gap {ref['gap']:.2e}): index parity unpinned")
    assert int(host(r.best_idx)[0]) == ref["best_idx"]
    assert np.array_equal(host(r.s_best).view(np.uint16), ref["s_best"].view(np.uint16))
    p = awq.quantize_pack(to_dev(W), r.s_best)
    qw, sc, zb = packed_host(p)
    assert np.array_equal(qw, ref["qweight"]) and np.array_equal(zb, ref["zeros"])
    assert np.array_equal(sc.view(np.uint16), ref["scales"].view(np.uint16))
    return ref


@pytest.mark.parametrize("lo,hi", [(-6, 6), (-10, 10), (-14, 12)])
def test_search_log_uniform_channel_magnitudes(lo, hi):
    """Channel magnitudes log-uniform over 2^lo .. 2^hi: at alpha = 0.95 the scales span
    2^11 .. 2^25 (max s / min s; |x| stays below 65504), with two row tiles and a ragged third."""
    T, N, K = 512, 300, 1024
    X = si.activations_wide(T, K, offset=hi, log2_lo=lo, log2_hi=hi)
    W = si.weights(N, K, offset=hi + 1)
    ref = _check_search(X, W)
    s = ref["s16"].astype(np.float64)
    assert s[19].max() / s[19].min() > 2.0 ** 10


def test_search_dead_and_outlier_channels():
    """Dead channels (all-zero activations: statistic floored at 2^-14) beside the x20
    outlier channels, plus near-dead ones at 1e-4 of the rest: the largest scale range
    of a realistic layer, over two 128-channel steps with no dead channel."""
    T, N, K = 512, 256, 1280
    X = si.activations(T, K, offset=31, channel_offset=K).astype(np.float32)
    g = np.random.default_rng(31)
    ch = g.permutation(np.arange(256, K))   # channels 0..255 stay ordinary
    X[:, ch[:6]] = 0.0
    X[:, ch[6:12]] *= np.float32(1e-4)
    X = X.astype(np.float16)
    W = si.weights(N, K, offset=32)
    _check_search(X, W)


@pytest.mark.parametrize("w_bit,group,zp", [(8, 128, True), (3, 64, True), (4, 32, False)])
def test_search_wide_range_format_variants(w_bit, group, zp):
    """The same wide range with 8-bit codes (smaller D, 500 x below the weights), 3-bit
    codes and small groups, symmetric codes."""
    T, N, K = 256, 160, 512
    X = si.activations_wide(T, K, offset=40 + w_bit, log2_lo=-8, log2_hi=8, n_zero=3)
    W = si.weights(N, K, offset=41)
    ref = oracle.search_scales(X, W, zero_point=zp, group=group, w_bit=w_bit)
    r = awq.search_scales(to_dev(X), to_dev(W), zero_point=zp, group_size=group, w_bit=w_bit)
    err = host(r.err)
    assert np.all(np.abs(err - ref["err"]) <= 1e-5 * ref["err"])
    if ref["gap"] >= 1e-5:
        assert int(host(r.best_idx)[0]) == ref["best_idx"]
