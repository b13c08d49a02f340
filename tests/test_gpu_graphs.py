"""Every entry point captured in a HIP graph and replayed.

The benchmark times graph replays, so each entry point must give, on every replay, what an
eager call gives on the same inputs. Per case: one eager call (loads the code objects),
capture, then several rounds of eager work in between: new input values written in place,
an eager reference call, a synchronization, the outputs poisoned, one replay, and a
bit-exact comparison of every output. The library records no memset and allocates
nothing, so nothing but its kernels is in the graphs.
"""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
import weight_only_bit_02_amd as awq
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

ROUNDS = 3


def _replay_matches_eager(run, update):
    """run() launches on the current stream and returns its output tensors; update(i)
    rewrites the inputs in place (eager work between replays)."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            outs = run()
        torch.cuda.synchronize()
        for i in range(ROUNDS):
            update(i)
            ref = [o.clone() for o in run()]
            torch.cuda.synchronize()
            for o in outs:
                o.view(torch.uint8).fill_(0xA5)  # a replay that writes nothing cannot pass
            graph.replay()
            torch.cuda.synchronize()
            for o, r in zip(outs, ref):
                assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), i
        del graph


def _refill(t, seed, std):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t.copy_((torch.randn(t.shape, generator=g, device=DEV) * std).to(t.dtype))


@pytest.mark.parametrize("w_bit,group", [(4, 128), (4, 32), (8, 64), (3, 128)])
def test_graph_pack_and_linear(w_bit, group):
    N, K = 384, 1152
    W = si.torch_weights(N, K, 11, DEV)
    s = (torch.rand(K, device=DEV) + 0.5).half()
    p = awq.alloc_packed(N, K, DEV, group, w_bit)
    x1 = si.torch_activations(1, K, 12, DEV)
    x16 = si.torch_activations(16, K, 13, DEV)
    x64 = si.torch_activations(64, K, 14, DEV)
    y1 = torch.empty((1, N), dtype=torch.float16, device=DEV)
    y16 = torch.empty((16, N), dtype=torch.float16, device=DEV)
    y64 = torch.empty((64, N), dtype=torch.float16, device=DEV)
    h1 = torch.empty((1, N // 2), dtype=torch.float16, device=DEV)

    def run():
        awq.quantize_pack(W, s, out=p, group_size=group, w_bit=w_bit)
        awq.linear_w4a16(x1, p, out=y1)
        awq.linear_w4a16(x16, p, out=y16)
        awq.linear_w4a16(x64, p, out=y64)
        awq.linear_w4a16_gated_silu(x1, p, out=h1)
        return [p.qweight, p.scales, p.zeros, y1, y16, y64, h1]

    def update(i):
        _refill(W, 100 + i, 0.02)
        for j, x in enumerate((x1, x16, x64)):
            _refill(x, 200 + 10 * i + j, 1.0)

    _replay_matches_eager(run, update)


@pytest.mark.parametrize("group", [128, 64])
def test_graph_search_clip_stats_fold(group):
    T, N, K = 256, 256, 1024
    X = si.torch_activations(T, K, 21, DEV)
    W = si.torch_weights(N, K, 22, DEV)
    ws = awq.SearchWorkspace(T, N, K, DEV)
    res = awq.search_scales(X, W, workspace=ws, group_size=group)
    nb = torch.empty(K, dtype=torch.float16, device=DEV)
    _refill(nb, 7, 1.0)
    nb_out = torch.empty_like(nb)

    def run():
        act = awq.activation_stats(X)
        awq.search_scales(X, W, workspace=ws, out=res, group_size=group)
        idx, err = awq.clip_search(X, W, res.s_best, 200, 8, group_size=group)
        awq.apply_inverse_scale(nb, res.s_best, 1, out=nb_out)
        return [act, res.s_best, res.best_idx, res.err, res.s_grid, idx, err, nb_out]

    def update(i):
        _refill(X, 300 + i, 1.0)
        _refill(W, 400 + i, 0.02)

    _replay_matches_eager(run, update)
